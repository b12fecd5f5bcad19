"""Python binding of libfmask (mask-aware attention forward for MI355X).

Argument marshalling only: every step of the path (mask encoding, tile
classification, attention) runs in the HIP kernels of libfmask.so, called
through its C ABI (include/fmask.h).  PyTorch supplies device memory and the
current stream.  There is no CPU fallback: if the library is missing or a
call fails, an exception is raised.

    enc   = encode(spec)                      # spec: dict, see encode()
    tiles = classify(enc, dtype="bf16", d=128)
    o, lse = attn_fwd(q, k, v, enc, tiles)
"""

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfmask.so")

# status codes
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_HIP = 0, -1, -2, -3, -4
# families
FAMILIES = {
    "causal": 1, "document": 2, "causal_document": 3, "shared_question": 4, "band": 5,
    "tree": 6, "block_bitmap": 7, "selected_key": 8, "intervals": 9,
    "causal_bottom_right": 10, "varlen": 11, "dense": 12,
}
VARLEN_MODES = {"full": 0, "causal": 1, "causal_bottom_right": 2, "band": 3, "prefix": 4}
ENC_INTERVALS, ENC_BITMAP, ENC_SELECTED = 1, 2, 3
SKIP, PARTIAL, FULL = 0, 1, 2
DTYPES = {"f32": 0, "bf16": 1}
LIST_FULL_BIT = 0x80000000

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p


class MaskDesc(ctypes.Structure):
    _fields_ = [
        ("family", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("reserved0", ctypes.c_int32), ("sq", ctypes.c_int64), ("skv", ctypes.c_int64),
        ("cu_seg", _vp), ("n_seg", ctypes.c_int32), ("reserved1", ctypes.c_int32),
        ("pre_tokens", ctypes.c_int64), ("next_tokens", ctypes.c_int64),
        ("tree_parent", _vp), ("tree_prefix", ctypes.c_int32), ("tree_n", ctypes.c_int32),
        ("blk_state", _vp), ("blk_index", _vp), ("blk_bits", _vp), ("blk_pool_n", ctypes.c_int64),
        ("force_diag", ctypes.c_int32), ("reserved2", ctypes.c_int32),
        ("sel", _vp), ("sel_n", ctypes.c_int32), ("sel_cells", ctypes.c_int32),
        ("raw_intervals", _vp), ("cu_seg_k", _vp), ("seg_mode", _vp), ("seg_prefix", _vp),
        ("dense", _vp), ("dense_form", ctypes.c_int32), ("reserved3", ctypes.c_int32),
    ]


class Encoded(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("blk", ctypes.c_int32), ("sq", ctypes.c_int64), ("skv", ctypes.c_int64),
        ("intervals", _vp), ("blk_state", _vp), ("blk_index", _vp), ("blk_bits", _vp),
        ("blk_pool_count", _vp), ("nbq", ctypes.c_int64), ("nbk", ctypes.c_int64),
        ("pool_cap", ctypes.c_int64), ("sel_list", _vp), ("sel_count", _vp),
        ("sel_n", ctypes.c_int32), ("reserved0", ctypes.c_int32),
    ]


class Tiles(ctypes.Structure):
    _fields_ = [
        ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("nqt", ctypes.c_int32),
        ("nkt", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("reserved0", ctypes.c_int32), ("reserved1", ctypes.c_int32),
        ("state", _vp), ("list", _vp), ("count", _vp), ("order", _vp),
    ]


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("b", ctypes.c_int32), ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32), ("sq", ctypes.c_int64), ("skv", ctypes.c_int64),
        ("d", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("scale", ctypes.c_float), ("reserved1", ctypes.c_int32),
    ]


EXPORTS = ("fmask_encode_bytes", "fmask_encode", "fmask_classify_bytes", "fmask_classify",
           "fmask_attn_fwd", "fmask_attn_split_workspace_bytes", "fmask_attn_fwd_split",
           "fmask_attn_fwd_split_noalloc", "fmask_attn_blocks_workspace_bytes", "fmask_attn_fwd_blocks",
           "fmask_attn_bwd_workspace_bytes", "fmask_attn_bwd",
           "fmask_preferred_tile", "fmask_status_str", "fmask_last_error")

_lib = None


class FmaskError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libfmask status {status}: {msg}")
        self.status = status


def lib():
    """The loaded libfmask.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(python mask_aware_block_amd/build.py); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        L.fmask_encode_bytes.argtypes = [ctypes.POINTER(MaskDesc)]
        L.fmask_encode_bytes.restype = ctypes.c_size_t
        L.fmask_encode.argtypes = [ctypes.POINTER(MaskDesc), _vp, ctypes.c_size_t,
                                   ctypes.POINTER(Encoded), _vp]
        L.fmask_encode.restype = ctypes.c_int32
        L.fmask_classify_bytes.argtypes = [ctypes.POINTER(Encoded), ctypes.c_int32, ctypes.c_int32]
        L.fmask_classify_bytes.restype = ctypes.c_size_t
        L.fmask_classify.argtypes = [ctypes.POINTER(Encoded), ctypes.c_int32, ctypes.c_int32, _vp,
                                     ctypes.c_size_t, ctypes.POINTER(Tiles), _vp]
        L.fmask_classify.restype = ctypes.c_int32
        L.fmask_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), _vp, _vp, _vp, _vp, _vp,
                                     ctypes.POINTER(Encoded), ctypes.POINTER(Tiles), _vp]
        L.fmask_attn_fwd.restype = ctypes.c_int32
        L.fmask_attn_split_workspace_bytes.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(Encoded),
                                                       ctypes.c_int32]
        L.fmask_attn_split_workspace_bytes.restype = ctypes.c_size_t
        L.fmask_attn_fwd_split.argtypes = [ctypes.POINTER(AttnArgs), _vp, _vp, _vp, _vp, _vp,
                                           ctypes.POINTER(Encoded), ctypes.c_int32, _vp, ctypes.c_size_t, _vp]
        L.fmask_attn_fwd_split.restype = ctypes.c_int32
        L.fmask_attn_fwd_split_noalloc.argtypes = [ctypes.POINTER(AttnArgs), _vp, _vp, _vp, _vp, _vp,
                                                   ctypes.POINTER(Encoded), ctypes.c_int32, _vp]
        L.fmask_attn_fwd_split_noalloc.restype = ctypes.c_int32
        L.fmask_attn_blocks_workspace_bytes.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(Encoded)]
        L.fmask_attn_blocks_workspace_bytes.restype = ctypes.c_size_t
        L.fmask_attn_fwd_blocks.argtypes = [ctypes.POINTER(AttnArgs), _vp, _vp, _vp, _vp, _vp,
                                            ctypes.POINTER(Encoded), _vp, ctypes.c_size_t, _vp]
        L.fmask_attn_fwd_blocks.restype = ctypes.c_int32
        L.fmask_attn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(Tiles)]
        L.fmask_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.fmask_attn_bwd.argtypes = [ctypes.POINTER(AttnArgs)] + [_vp] * 10 + [
            ctypes.c_size_t, ctypes.POINTER(Encoded), ctypes.POINTER(Tiles), _vp]
        L.fmask_attn_bwd.restype = ctypes.c_int32
        L.fmask_preferred_tile.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           _c_i32p, _c_i32p]
        L.fmask_preferred_tile.restype = ctypes.c_int32
        L.fmask_status_str.argtypes = [ctypes.c_int32]
        L.fmask_status_str.restype = ctypes.c_char_p
        L.fmask_last_error.argtypes = []
        L.fmask_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status):
    if status != OK:
        L = lib()
        raise FmaskError(status, f"{L.fmask_status_str(status).decode()}: {L.fmask_last_error().decode()}")


def _torch():
    import torch
    return torch


def _stream_handle(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(x, dtype, device):
    """Contiguous device tensor of x (numpy dtype `dtype`)."""
    torch = _torch()
    if isinstance(x, torch.Tensor):
        return x.to(device).contiguous()
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=dtype))).to(device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def make_desc(spec, device="cuda"):
    """(MaskDesc, keep-alive list) for a mask spec dict.

    Spec keys: family (name), sq, skv, batch, heads, and per family: cu_seg,
    pre, next, tree_prefix, tree_parent, blk_state, blk_index, blk_bits,
    force_diag, sel, sel_cells, raw_intervals.  Host arrays (cu_seg,
    tree_parent) stay on the host; the others are copied to `device`.
    """
    d = MaskDesc()
    keep = []
    d.family = FAMILIES[spec["family"]]
    d.batch = int(spec.get("batch", 1))
    d.heads = int(spec.get("heads", 1))
    d.sq, d.skv = int(spec["sq"]), int(spec["skv"])
    if "cu_seg" in spec and spec["cu_seg"] is not None:
        cu = np.ascontiguousarray(np.asarray(spec["cu_seg"], dtype=np.int32))
        keep.append(cu)
        d.cu_seg = cu.ctypes.data
        d.n_seg = cu.size - 1
    d.pre_tokens = int(spec.get("pre") or 0)
    d.next_tokens = int(spec.get("next") or 0)
    if spec.get("tree_parent") is not None:
        par = np.ascontiguousarray(np.asarray(spec["tree_parent"], dtype=np.int32))
        keep.append(par)
        d.tree_parent = par.ctypes.data
        d.tree_n = par.size
        d.tree_prefix = int(spec["tree_prefix"])
    if spec.get("blk_state") is not None:
        st = _dev(spec["blk_state"], np.uint8, device)
        ix = _dev(spec["blk_index"], np.int32, device)
        bits = np.ascontiguousarray(np.asarray(spec["blk_bits"], dtype=np.uint64))
        bt = _dev(bits.view(np.int64), np.int64, device) if bits.size else None
        keep += [st, ix, bt]
        d.blk_state, d.blk_index = st.data_ptr(), ix.data_ptr()
        d.blk_bits = bt.data_ptr() if bt is not None else None
        d.blk_pool_n = bits.shape[0] if bits.size else 0
        d.force_diag = int(bool(spec.get("force_diag", False)))
    if spec.get("sel") is not None:
        sel = _dev(spec["sel"], np.int32, device)
        keep.append(sel)
        d.sel = sel.data_ptr()
        d.sel_n = sel.shape[-1]
        d.sel_cells = int(spec.get("sel_cells", 32))
    if spec["family"] == "varlen":
        cq = np.ascontiguousarray(np.asarray(spec["cu_q"], dtype=np.int32))
        ck = np.ascontiguousarray(np.asarray(spec["cu_k"], dtype=np.int32))
        md = np.ascontiguousarray(np.asarray([VARLEN_MODES[m] if isinstance(m, str) else int(m)
                                              for m in spec["seg_mode"]], dtype=np.int32))
        keep += [cq, ck, md]
        d.cu_seg, d.n_seg = cq.ctypes.data, cq.size - 1
        d.cu_seg_k, d.seg_mode = ck.ctypes.data, md.ctypes.data
        if spec.get("seg_prefix") is not None:
            pf = np.ascontiguousarray(np.asarray(spec["seg_prefix"], dtype=np.int32))
            keep.append(pf)
            d.seg_prefix = pf.ctypes.data
    if spec["family"] == "dense":
        dn = _dev(spec["dense"], np.uint8, device)
        keep.append(dn)
        d.dense = dn.data_ptr()
        d.dense_form = {None: 0, "auto": 0, "intervals": ENC_INTERVALS, "bitmap": ENC_BITMAP}[
            spec.get("dense_form")]
    if spec.get("raw_intervals") is not None:
        raw = _dev(spec["raw_intervals"], np.int32, device)
        keep.append(raw)
        d.raw_intervals = raw.data_ptr()
    return d, keep


class Encoding:
    """Canonical encoding on the device (owns its buffer)."""

    def __init__(self, struct, buf, keep):
        self.struct, self.buf, self._keep = struct, buf, keep

    @property
    def kind(self):
        return self.struct.kind

    def _view(self, ptr, nbytes, dtype, shape):
        torch = _torch()
        off = ptr - self.buf.data_ptr()
        return self.buf[off: off + nbytes].view(dtype).reshape(shape)

    def intervals(self):
        torch = _torch()
        e = self.struct
        shape = (e.batch, e.heads, 4, e.skv)
        return self._view(e.intervals, 4 * int(np.prod(shape)), torch.int32, shape)

    def bitmap(self):
        """(state, index, pool words [count][64] as int64, count)."""
        torch = _torch()
        e = self.struct
        shape = (e.batch, e.heads, e.nbq, e.nbk)
        n = int(np.prod(shape))
        st = self._view(e.blk_state, n, torch.uint8, shape)
        ix = self._view(e.blk_index, 4 * n, torch.int32, shape)
        cnt = int(self._view(e.blk_pool_count, 4, torch.int32, (1,)).item())
        bits = self._view(e.blk_bits, 8 * 64 * cnt, torch.int64, (cnt, 64))
        return st, ix, bits, cnt

    def lists(self):
        torch = _torch()
        e = self.struct
        shape = (e.batch, e.sq, e.sel_n)
        ls = self._view(e.sel_list, 4 * int(np.prod(shape)), torch.int32, shape)
        cn = self._view(e.sel_count, 4 * e.batch * e.sq, torch.int32, (e.batch, e.sq))
        return ls, cn


class MaskInput:
    """A mask description with its device-side inputs already uploaded."""

    def __init__(self, spec, device="cuda"):
        self.desc, self.keep = make_desc(spec, device)


def encode(spec, device="cuda", stream=None, out=None):
    """Run the mask encoder (fmask_encode) on the device.

    spec: a mask spec dict (see make_desc) or a MaskInput.  out: optional uint8
    device buffer to hold the encoding (reused when large enough, e.g. across
    steps; the returned Encoding views it).
    """
    torch = _torch()
    L = lib()
    if isinstance(spec, MaskInput):
        desc, keep = spec.desc, [spec]
    else:
        desc, keep = make_desc(spec, device)
    nbytes = L.fmask_encode_bytes(ctypes.byref(desc))
    if nbytes == 0:
        _check(L.fmask_encode(ctypes.byref(desc), None, 0, ctypes.byref(Encoded()), None))
    if out is not None and out.dtype == torch.uint8 and out.is_cuda and out.numel() >= nbytes:
        buf = out
    else:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    enc = Encoded()
    _check(L.fmask_encode(ctypes.byref(desc), _ptr(buf), buf.numel(), ctypes.byref(enc), _stream_handle(stream)))
    keep.append(desc)
    return Encoding(enc, buf, keep)


_preferred = {}


def preferred_tile(dtype, d, kind):
    key = (id(lib()), dtype, int(d), int(kind))
    if key not in _preferred:
        bm, bn = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().fmask_preferred_tile(DTYPES[dtype], int(d), int(kind), ctypes.byref(bm), ctypes.byref(bn)))
        _preferred[key] = (bm.value, bn.value)
    return _preferred[key]


class TileTable:
    """Tile states, compact lists, counts and order on the device."""

    def __init__(self, struct, buf, enc):
        self.struct, self.buf, self.enc = struct, buf, enc

    def _view(self, ptr, nbytes, dtype, shape):
        off = ptr - self.buf.data_ptr()
        return self.buf[off: off + nbytes].view(dtype).reshape(shape)

    def arrays(self):
        torch = _torch()
        t = self.struct
        rows = t.batch * t.heads * t.nqt
        st = self._view(t.state, rows * t.nkt, torch.uint8, (t.batch, t.heads, t.nqt, t.nkt))
        ls = self._view(t.list, 4 * rows * t.nkt, torch.int32, (t.batch, t.heads, t.nqt, t.nkt))
        cn = self._view(t.count, 4 * rows, torch.int32, (t.batch, t.heads, t.nqt))
        od = self._view(t.order, 4 * rows, torch.int32, (rows,))
        return st, ls, cn, od



def classify(enc, bm=None, bn=None, dtype="bf16", d=128, stream=None, out=None):
    """Run the tile classifier (fmask_classify) at bm x bn (default: the kernel's
    tile).  out: optional uint8 device buffer for the table (reused when large
    enough)."""
    torch = _torch()
    L = lib()
    if bm is None or bn is None:
        bm, bn = preferred_tile(dtype, d, enc.kind)
    nbytes = L.fmask_classify_bytes(ctypes.byref(enc.struct), int(bm), int(bn))
    if nbytes == 0:
        _check(L.fmask_classify(ctypes.byref(enc.struct), int(bm), int(bn), None, 0,
                                ctypes.byref(Tiles()), None))
    if out is not None and out.dtype == torch.uint8 and out.is_cuda and out.numel() >= nbytes:
        buf = out
    else:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=enc.buf.device)
    t = Tiles()
    _check(L.fmask_classify(ctypes.byref(enc.struct), int(bm), int(bn), _ptr(buf), buf.numel(),
                            ctypes.byref(t), _stream_handle(stream)))
    return TileTable(t, buf, enc)


def attn_args(q, k, v, o, scale):
    torch = _torch()
    a = AttnArgs()
    if q.dtype == torch.bfloat16:
        a.dtype = DTYPES["bf16"]
    elif q.dtype == torch.float32:
        a.dtype = DTYPES["f32"]
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    B, Hq, Sq, D = q.shape
    a.b, a.hq, a.hkv = B, Hq, k.shape[1]
    a.sq, a.skv, a.d = Sq, k.shape[2], D
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o)):
        if t.stride(3) != 1:
            raise ValueError(f"{name}: last dimension must be contiguous")
        getattr(a, name)[:] = (t.stride(0), t.stride(1), t.stride(2))
    a.scale = float(scale)
    return a


def attn_fwd(q, k, v, enc, tiles=None, scale=None, out=None, lse=None, want_lse=True, stream=None):
    """Masked attention forward (fmask_attn_fwd).  q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D]."""
    torch = _torch()
    L = lib()
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    a = attn_args(q, k, v, out, scale)
    st = L.fmask_attn_fwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                          ctypes.byref(enc.struct),
                          ctypes.byref(tiles.struct) if tiles is not None else None,
                          _stream_handle(stream))
    _check(st)
    return out, lse


def attn_fwd_split(q, k, v, enc, splits=0, scale=None, out=None, lse=None, workspace=None, stream=None):
    """Few-query form of attn_fwd for selected-key lists (fmask_attn_fwd_split):
    each list is split over `splits` workgroups (0 = automatic) and merged."""
    torch = _torch()
    L = lib()
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    a = attn_args(q, k, v, out, scale)
    nbytes = L.fmask_attn_split_workspace_bytes(ctypes.byref(a), ctypes.byref(enc.struct), int(splits))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = L.fmask_attn_fwd_split(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                ctypes.byref(enc.struct), int(splits), _ptr(workspace), workspace.numel(),
                                _stream_handle(stream))
    _check(st)
    return out, lse


SPLIT_SCRATCH_BYTES = 16 << 20  # FMASK_SPLIT_SCRATCH_BYTES


def attn_fwd_split_noalloc(q, k, v, enc, splits=0, scale=None, out=None, lse=None, stream=None):
    """attn_fwd_split with the partial states in the library's own per-GPU
    scratch (fmask_attn_fwd_split_noalloc): nothing is allocated, so out and
    lse must be given when the caller cannot allocate either."""
    torch = _torch()
    L = lib()
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    a = attn_args(q, k, v, out, scale)
    st = L.fmask_attn_fwd_split_noalloc(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                        ctypes.byref(enc.struct), int(splits), _stream_handle(stream))
    _check(st)
    return out, lse


def attn_blocks_workspace_bytes(q, k, v, enc):
    """Bytes of device workspace attn_fwd_blocks needs (fmask_attn_blocks_workspace_bytes)."""
    return lib().fmask_attn_blocks_workspace_bytes(ctypes.byref(attn_args(q, k, v, q, 1.0)),
                                                   ctypes.byref(enc.struct))


def attn_fwd_blocks(q, k, v, enc, scale=None, out=None, lse=None, workspace=None, stream=None):
    """Block-major form of attn_fwd for selected-key lists (fmask_attn_fwd_blocks):
    each listed block's K and V are read once per K/V head and scored against
    the queries that name it; the per-entry partial states are merged per query.
    workspace: optional uint8 device buffer of attn_blocks_workspace_bytes bytes."""
    torch = _torch()
    L = lib()
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    a = attn_args(q, k, v, out, scale)
    nbytes = L.fmask_attn_blocks_workspace_bytes(ctypes.byref(a), ctypes.byref(enc.struct))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = L.fmask_attn_fwd_blocks(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 ctypes.byref(enc.struct), _ptr(workspace), workspace.numel(),
                                 _stream_handle(stream))
    _check(st)
    return out, lse


def attn_bwd_workspace_bytes(q, k, v, out, tiles):
    """Bytes of device workspace attn_bwd needs (fmask_attn_bwd_workspace_bytes)."""
    return lib().fmask_attn_bwd_workspace_bytes(ctypes.byref(attn_args(q, k, v, out, 1.0)),
                                                ctypes.byref(tiles.struct))


def attn_bwd(q, k, v, out, lse, dout, enc, tiles, scale=None, dq=None, dk=None, dv=None,
             workspace=None, stream=None):
    """Gradient of the masked attention forward (fmask_attn_bwd).

    q, k, v, the forward's out and lse, and the output gradient dout (laid out
    like out).  Returns (dq, dk, dv) shaped like q, k, v.
    """
    torch = _torch()
    L = lib()
    if scale is None:
        scale = 1.0 / float(q.shape[-1]) ** 0.5
    if dout.stride() != out.stride():
        raise ValueError("dout must be laid out like out")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("dq, dk, dv must be laid out like q, k, v")
    a = attn_args(q, k, v, out, scale)
    nbytes = L.fmask_attn_bwd_workspace_bytes(ctypes.byref(a), ctypes.byref(tiles.struct))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = L.fmask_attn_bwd(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                          ctypes.byref(enc.struct), ctypes.byref(tiles.struct), _stream_handle(stream))
    _check(st)
    return dq, dk, dv
