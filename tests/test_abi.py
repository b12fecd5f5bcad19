"""C-ABI checks that need no GPU: libfmask.so loads, exports every function
include/fmask.h declares, its structs have the layout the binding assumes, and
host-detectable errors come back as status codes before anything is launched."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import mask_aware_block_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmask.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_]\w*\s*\**\s*(fmask_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for must in ("fmask_encode", "fmask_classify", "fmask_attn_fwd", "fmask_encode_bytes",
                 "fmask_classify_bytes"):
        assert must in names
    assert set(names) == set(fm.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = fm.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", fm.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "sizes.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "fmask.h"\n'
        "int main(void) {\n"
        '  printf("%zu %zu %zu %zu\\n", sizeof(fmask_mask_desc), sizeof(fmask_encoded),'
        " sizeof(fmask_tiles), sizeof(fmask_attn_args));\n"
        '  printf("%zu %zu %zu %zu\\n", offsetof(fmask_mask_desc, raw_intervals),'
        " offsetof(fmask_encoded, sel_n), offsetof(fmask_tiles, order), offsetof(fmask_attn_args, scale));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "sizes"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    sizes = [int(x) for x in lines[0].split()]
    offs = [int(x) for x in lines[1].split()]
    assert sizes == [ctypes.sizeof(fm.MaskDesc), ctypes.sizeof(fm.Encoded), ctypes.sizeof(fm.Tiles),
                     ctypes.sizeof(fm.AttnArgs)]
    assert offs == [fm.MaskDesc.raw_intervals.offset, fm.Encoded.sel_n.offset, fm.Tiles.order.offset,
                    fm.AttnArgs.scale.offset]


def test_status_strings_and_preferred_tiles():
    L = fm.lib()
    for s in (fm.OK, fm.ERR_INVALID, fm.ERR_UNSUPPORTED, fm.ERR_CAPACITY, fm.ERR_HIP):
        assert L.fmask_status_str(s)
    assert fm.preferred_tile("bf16", 128, fm.ENC_INTERVALS) == (128, 64)
    assert fm.preferred_tile("bf16", 128, fm.ENC_BITMAP) == (128, 64)
    assert fm.preferred_tile("f32", 64, fm.ENC_INTERVALS) == (64, 64)
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    assert L.fmask_preferred_tile(1, 96, fm.ENC_INTERVALS, ctypes.byref(bm), ctypes.byref(bn)) == fm.ERR_UNSUPPORTED
    assert L.fmask_preferred_tile(1, 128, fm.ENC_SELECTED, ctypes.byref(bm), ctypes.byref(bn)) == fm.ERR_INVALID


def _desc(**kw):
    d = fm.MaskDesc()
    d.family, d.batch, d.heads = kw.pop("family"), kw.pop("batch", 1), kw.pop("heads", 1)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_encode_bytes_and_host_validation():
    L = fm.lib()
    ok = _desc(family=1, sq=1000, skv=1000)
    assert L.fmask_encode_bytes(ctypes.byref(ok)) >= 4 * 1000 * 4
    bad_sizes = _desc(family=1, sq=-1, skv=10)
    assert L.fmask_encode_bytes(ctypes.byref(bad_sizes)) == 0
    cu = np.array([0, 64, 32, 256], dtype=np.int32)  # not increasing
    doc = _desc(family=3, sq=256, skv=256, cu_seg=cu.ctypes.data, n_seg=3)
    assert L.fmask_encode_bytes(ctypes.byref(doc)) == 0
    enc = fm.Encoded()
    st = L.fmask_encode(ctypes.byref(doc), None, 0, ctypes.byref(enc), None)
    assert st == fm.ERR_INVALID and L.fmask_last_error()
    cu_short = np.array([0, 64, 200], dtype=np.int32)  # last offset != sq
    doc2 = _desc(family=3, sq=256, skv=256, cu_seg=cu_short.ctypes.data, n_seg=2)
    assert L.fmask_encode(ctypes.byref(doc2), None, 0, ctypes.byref(enc), None) == fm.ERR_INVALID
    par = np.array([-1, 0, 2], dtype=np.int32)  # parent not before child
    tree = _desc(family=6, sq=67, skv=67, tree_parent=par.ctypes.data, tree_prefix=64, tree_n=3)
    assert L.fmask_encode(ctypes.byref(tree), None, 0, ctypes.byref(enc), None) == fm.ERR_INVALID
    unknown = _desc(family=42, sq=8, skv=8)
    assert L.fmask_encode(ctypes.byref(unknown), None, 0, ctypes.byref(enc), None) == fm.ERR_INVALID
    # valid description, but no output buffer / too small: rejected before any launch
    assert L.fmask_encode(ctypes.byref(ok), None, 0, ctypes.byref(enc), None) == fm.ERR_INVALID
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: the size check fails first
    assert L.fmask_encode(ctypes.byref(ok), fake, 16, ctypes.byref(enc), None) == fm.ERR_CAPACITY


def test_classify_and_attn_host_validation():
    L = fm.lib()
    enc = fm.Encoded()
    enc.kind, enc.batch, enc.heads, enc.sq, enc.skv = fm.ENC_INTERVALS, 1, 1, 512, 512
    enc.intervals = 1 << 20
    assert L.fmask_classify_bytes(ctypes.byref(enc), 128, 64) > 0
    assert L.fmask_classify_bytes(ctypes.byref(enc), 100, 64) == 0  # not a multiple of 16
    assert L.fmask_classify_bytes(ctypes.byref(enc), 512, 64) == 0  # above 256
    tiles = fm.Tiles()
    fake = ctypes.c_void_p(1 << 20)
    assert L.fmask_classify(ctypes.byref(enc), 128, 64, fake, 16, ctypes.byref(tiles), None) == fm.ERR_CAPACITY
    enc_b = fm.Encoded()
    enc_b.kind, enc_b.batch, enc_b.heads, enc_b.sq, enc_b.skv = fm.ENC_BITMAP, 1, 1, 512, 512
    assert L.fmask_classify_bytes(ctypes.byref(enc_b), 96, 64) == 0  # bitmap tiles: multiples of 64

    a = fm.AttnArgs()
    a.dtype, a.b, a.hq, a.hkv, a.sq, a.skv, a.d, a.scale = 1, 1, 6, 4, 512, 512, 128, 0.08
    p = ctypes.c_void_p(1 << 20)
    assert L.fmask_attn_fwd(ctypes.byref(a), p, p, p, p, None, ctypes.byref(enc), ctypes.byref(tiles),
                            None) == fm.ERR_INVALID  # hq % hkv != 0
    a.hq = 8
    a.sq = 256
    assert L.fmask_attn_fwd(ctypes.byref(a), p, p, p, p, None, ctypes.byref(enc), ctypes.byref(tiles),
                            None) == fm.ERR_INVALID  # differs from the encoding
    a.sq, a.dtype = 512, 7
    assert L.fmask_attn_fwd(ctypes.byref(a), p, p, p, p, None, ctypes.byref(enc), ctypes.byref(tiles),
                            None) == fm.ERR_UNSUPPORTED
    a.dtype = 1
    assert L.fmask_attn_fwd(ctypes.byref(a), None, p, p, p, None, ctypes.byref(enc), ctypes.byref(tiles),
                            None) == fm.ERR_INVALID  # null tensor


def test_split_backward_varlen_dense_host_validation():
    """The entry points added for decode, backward, varlen and dense input
    reject bad arguments with status codes before any launch."""
    L = fm.lib()
    p = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails a host check first
    a = fm.AttnArgs()
    a.dtype, a.b, a.hq, a.hkv, a.sq, a.skv, a.d, a.scale = 1, 1, 8, 2, 512, 512, 128, 0.08
    # split decode: SELECTED encodings only, splits in [0, 64]
    iv_enc = fm.Encoded()
    iv_enc.kind, iv_enc.batch, iv_enc.heads, iv_enc.sq, iv_enc.skv = fm.ENC_INTERVALS, 1, 1, 512, 512
    assert L.fmask_attn_fwd_split(ctypes.byref(a), p, p, p, p, None, ctypes.byref(iv_enc), 0, None, 0,
                                  None) == fm.ERR_UNSUPPORTED
    sel = fm.Encoded()
    sel.kind, sel.batch, sel.heads, sel.sq, sel.skv, sel.sel_n = fm.ENC_SELECTED, 1, 1, 512, 512, 64
    assert L.fmask_attn_fwd_split(ctypes.byref(a), p, p, p, p, None, ctypes.byref(sel), 65, None, 0,
                                  None) == fm.ERR_INVALID
    # no-allocation split form: null arguments are refused before the scratch lookup
    assert L.fmask_attn_fwd_split_noalloc(None, p, p, p, p, None, ctypes.byref(sel), 0, None) == fm.ERR_INVALID
    assert L.fmask_attn_fwd_split_noalloc(ctypes.byref(a), p, p, p, p, None, None, 0, None) == fm.ERR_INVALID
    assert L.fmask_attn_split_workspace_bytes(ctypes.byref(a), ctypes.byref(iv_enc), 4) == 0
    assert L.fmask_attn_split_workspace_bytes(ctypes.byref(a), ctypes.byref(sel), 4) > 0
    # block-major selected form: SELECTED encodings only, a workspace of at least the queried size
    assert L.fmask_attn_blocks_workspace_bytes(ctypes.byref(a), ctypes.byref(iv_enc)) == 0
    sel.blk = 32
    need_b = L.fmask_attn_blocks_workspace_bytes(ctypes.byref(a), ctypes.byref(sel))
    assert need_b >= 512 * 64 * 8 * (2 * 128 + 8)
    assert L.fmask_attn_fwd_blocks(ctypes.byref(a), p, p, p, p, None, ctypes.byref(iv_enc), p, need_b,
                                   None) == fm.ERR_UNSUPPORTED
    assert L.fmask_attn_fwd_blocks(ctypes.byref(a), p, p, p, p, None, ctypes.byref(sel), p, need_b - 256,
                                   None) == fm.ERR_CAPACITY
    assert L.fmask_attn_fwd_blocks(None, p, p, p, p, None, ctypes.byref(sel), p, need_b, None) == fm.ERR_INVALID
    assert L.fmask_attn_fwd_blocks(ctypes.byref(a), p, p, p, p, None, ctypes.byref(sel), None, need_b,
                                   None) == fm.ERR_INVALID
    # a hand-filled encoding with lists past FMASK_MAX_SEL_N (the merge has one lane per entry)
    sel.sel_n = 65
    assert L.fmask_attn_blocks_workspace_bytes(ctypes.byref(a), ctypes.byref(sel)) == 0
    assert L.fmask_attn_fwd_blocks(ctypes.byref(a), p, p, p, p, None, ctypes.byref(sel), p, need_b,
                                   None) == fm.ERR_INVALID
    assert b"sel_n" in L.fmask_last_error()
    sel.sel_n = 64
    # backward: bf16 only, 128 x 64 tables, workspace at least the queried size
    t = fm.Tiles()
    t.bm, t.bn, t.nqt, t.nkt, t.batch, t.heads = 128, 64, 4, 8, 1, 1
    need = L.fmask_attn_bwd_workspace_bytes(ctypes.byref(a), ctypes.byref(t))
    assert need >= 8 * 512 * 8
    args = [ctypes.byref(a)] + [p] * 4 + [ctypes.cast(p, ctypes.c_void_p)] + [p] * 4
    assert L.fmask_attn_bwd(*args, p, need, ctypes.byref(iv_enc), ctypes.byref(t), None) == fm.ERR_INVALID
    assert b"interval array" in L.fmask_last_error()  # a hand-filled encoding without its mask data
    iv_enc.intervals = p.value
    assert L.fmask_attn_bwd(*args, p, need - 16, ctypes.byref(iv_enc), ctypes.byref(t), None) == fm.ERR_CAPACITY
    # null tensor pointers are refused unless their sequence is empty
    nargs = [ctypes.byref(a), None] + [p] * 3 + [ctypes.cast(p, ctypes.c_void_p)] + [p] * 4
    assert L.fmask_attn_bwd(*nargs, p, need, ctypes.byref(iv_enc), ctypes.byref(t), None) == fm.ERR_INVALID
    assert b"null tensor pointer" in L.fmask_last_error()
    assert L.fmask_attn_fwd(ctypes.byref(a), p, None, p, p, None, ctypes.byref(iv_enc), ctypes.byref(t),
                            None) == fm.ERR_INVALID
    t64 = fm.Tiles()
    t64.bm, t64.bn, t64.nqt, t64.nkt, t64.batch, t64.heads = 64, 64, 8, 8, 1, 1
    assert L.fmask_attn_bwd(*args, p, need, ctypes.byref(iv_enc), ctypes.byref(t64), None) == fm.ERR_UNSUPPORTED
    a.dtype = 0
    assert L.fmask_attn_bwd(*args, p, need, ctypes.byref(iv_enc), ctypes.byref(t), None) == fm.ERR_UNSUPPORTED
    a.dtype = 1
    assert L.fmask_attn_bwd(*args, p, need, ctypes.byref(sel), ctypes.byref(t), None) == fm.ERR_UNSUPPORTED
    # a bitmap encoding is checked against the block grid that sq and skv imply (8 x 8 blocks of 64)
    bmp = fm.Encoded()
    bmp.kind, bmp.batch, bmp.heads, bmp.sq, bmp.skv, bmp.blk = fm.ENC_BITMAP, 1, 1, 512, 512, 64
    bmp.blk_state = bmp.blk_index = bmp.blk_bits = bmp.blk_pool_count = p.value
    for nbq, nbk, blk in ((7, 8, 64), (8, 9, 64), (8, 8, 32)):
        bmp.nbq, bmp.nbk, bmp.blk = nbq, nbk, blk
        assert L.fmask_attn_bwd(*args, p, need, ctypes.byref(bmp), ctypes.byref(t), None) == fm.ERR_INVALID
        assert L.fmask_attn_fwd(ctypes.byref(a), p, p, p, p, None, ctypes.byref(bmp), ctypes.byref(t),
                                None) == fm.ERR_INVALID
        assert b"block grid" in L.fmask_last_error()
        assert L.fmask_classify(ctypes.byref(bmp), 128, 64, p, 1 << 30, ctypes.byref(fm.Tiles()),
                                None) == fm.ERR_INVALID
    bmp.nbq, bmp.nbk, bmp.blk = 8, 8, 64
    bmp.blk_bits = None
    assert L.fmask_attn_bwd(*args, p, need, ctypes.byref(bmp), ctypes.byref(t), None) == fm.ERR_INVALID
    assert b"bitmap array" in L.fmask_last_error()
    bmp.blk_bits = p.value
    assert L.fmask_attn_bwd(*args, p, need - 16, ctypes.byref(bmp), ctypes.byref(t), None) == fm.ERR_CAPACITY
    # varlen: segment lengths must add up, modes must be known
    enc = fm.Encoded()
    cu = np.array([0, 100, 300], dtype=np.int32)
    cuk = np.array([0, 50, 260], dtype=np.int32)  # ends at 260, skv is 300
    md = np.array([1, 2], dtype=np.int32)
    vl = _desc(family=fm.FAMILIES["varlen"], sq=300, skv=300, cu_seg=cu.ctypes.data, cu_seg_k=cuk.ctypes.data,
               seg_mode=md.ctypes.data, n_seg=2)
    assert L.fmask_encode(ctypes.byref(vl), None, 0, ctypes.byref(enc), None) == fm.ERR_INVALID
    assert b"end at sq and skv" in L.fmask_last_error()
    cuk_ok = np.array([0, 50, 300], dtype=np.int32)
    md_bad = np.array([1, 9], dtype=np.int32)
    vl2 = _desc(family=fm.FAMILIES["varlen"], sq=300, skv=300, cu_seg=cu.ctypes.data, cu_seg_k=cuk_ok.ctypes.data,
                seg_mode=md_bad.ctypes.data, n_seg=2)
    assert L.fmask_encode(ctypes.byref(vl2), None, 0, ctypes.byref(enc), None) == fm.ERR_INVALID
    assert b"not a varlen mode" in L.fmask_last_error()
    # dense: the mask pointer and a known form are required
    dn = _desc(family=fm.FAMILIES["dense"], sq=64, skv=64)
    assert L.fmask_encode(ctypes.byref(dn), None, 0, ctypes.byref(enc), None) == fm.ERR_INVALID
    dn2 = _desc(family=fm.FAMILIES["dense"], sq=64, skv=64, dense=1 << 20, dense_form=fm.ENC_SELECTED)
    assert L.fmask_encode(ctypes.byref(dn2), None, 0, ctypes.byref(enc), None) == fm.ERR_INVALID
    assert b"dense_form" in L.fmask_last_error()
