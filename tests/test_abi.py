"""C ABI on the host: the library loads, exports every declared entry point, and
rejects bad arguments before touching the GPU (no compute call runs here)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import token_sparse_attention_rel_amd as tsa
from token_sparse_attention_rel_amd import _binding as B

A = 0x10000  # a 16-byte aligned fake device address (never dereferenced)
U = 0x10001  # misaligned


def declared_functions(root):
    text = open(os.path.join(root, "include", "tsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(root):
    names = declared_functions(root)
    assert len(names) >= 10
    h = ctypes.CDLL(B.lib_path())
    for name in names:
        assert hasattr(h, name), name
    assert set(names) == set(B._SIGNATURES)


def test_version_and_status_strings():
    assert tsa.abi_version() == 7
    assert tsa.status_string(0) == "ok"
    assert "shape" in tsa.status_string(B.ERR_SHAPE)
    assert tsa.status_string(99) == "unknown status"
    assert tsa.select_workspace_bytes(32760) >= 0


L = None


def lib():
    return B.lib()


def select(**kw):
    a = dict(x_cur=A, x_ref=None, off=0, n=64, dim=64, dt=B.BF16, kind=B.SCORE_REL_L1,
             mode=B.SELECT_TOPK, k=8, tau=0.0, aux=None, step=0, scores=A, mask=A, idx=A, pidx=A,
             na=A, ws=None, wsb=0)
    a.update(kw)
    return lib().tsa_select_active(a["x_cur"], a["x_ref"], a["off"], a["n"], a["dim"], a["dt"],
                                   a["kind"], a["mode"], a["k"], a["tau"], a["aux"], a["step"],
                                   a["scores"], a["mask"], a["idx"], a["pidx"], a["na"], a["ws"],
                                   a["wsb"], None)


def test_select_validation():
    assert select(n=0, k=0) == B.OK  # nothing to do, nothing launched
    assert select(mode=7) == B.ERR_INVALID_ARG
    assert select(kind=5) == B.ERR_INVALID_ARG
    assert select(dt=9) == B.ERR_DTYPE
    assert select(x_cur=None) == B.ERR_INVALID_ARG
    assert select(scores=None) == B.ERR_INVALID_ARG
    assert select(mask=None) == B.ERR_INVALID_ARG
    assert select(idx=None) == B.ERR_INVALID_ARG
    assert select(na=None) == B.ERR_INVALID_ARG
    assert select(k=65) == B.ERR_SHAPE
    assert select(k=-1) == B.ERR_SHAPE
    assert select(n=-1) == B.ERR_SHAPE
    assert select(n=1 << 31) == B.ERR_SHAPE
    assert select(dim=12) == B.ERR_SHAPE
    assert select(x_cur=U) == B.ERR_ALIGNMENT
    assert select(x_ref=U) == B.ERR_ALIGNMENT
    assert select(mode=B.SELECT_THRESHOLD, tau=float("nan")) == B.ERR_INVALID_ARG
    assert select(mode=B.SELECT_MASK, aux=None) == B.ERR_INVALID_ARG
    assert select(mode=B.SELECT_SCHEDULE, aux=A, step=-1) == B.ERR_SHAPE
    # MASK / SCHEDULE need no token rows and no scores
    assert select(mode=B.SELECT_MASK, aux=A, x_cur=None, scores=None, n=0) == B.OK


def qkv(**kw):
    a = dict(x=A, dt=B.BF16, nx=64, rows=A, n=16, dim=64, w=A, q=A, k=A, v=A, cache=0, ncache=0,
             eps=None, off=0, sigma=0.0)
    a.update(kw)
    return lib().tsa_qkv_active(a["x"], a["dt"], a["nx"], a["rows"], a["n"], a["dim"], a["w"],
                                a["q"], a["k"], a["v"], a["cache"], a["ncache"], a["eps"], a["off"],
                                a["sigma"], None)


def test_qkv_validation():
    assert qkv(n=0) == B.OK
    assert qkv(x=None) == B.ERR_INVALID_ARG
    assert qkv(w=None) == B.ERR_INVALID_ARG
    assert qkv(k=None) == B.ERR_INVALID_ARG
    assert qkv(dt=5) == B.ERR_DTYPE
    assert qkv(dt=B.F32, eps=A) == B.ERR_DTYPE
    assert qkv(dim=96) == B.ERR_SHAPE  # not a multiple of 64
    assert qkv(rows=None, n=65) == B.ERR_SHAPE
    assert qkv(cache=1, rows=None) == B.ERR_INVALID_ARG
    assert qkv(w=U) == B.ERR_ALIGNMENT
    assert qkv(eps=A, sigma=float("nan")) == B.ERR_INVALID_ARG
    assert qkv(rows=A + 2) == B.ERR_ALIGNMENT
    # token rows of 2 GiB and more are accepted (64-bit row addresses); n = 0 launches nothing
    assert qkv(nx=1 << 20, dim=1024, n=0) == B.OK
    assert qkv(nx=(1 << 31) - 1, dim=4096, n=0) == B.OK
    assert qkv(dim=19008) == B.ERR_SHAPE  # the weight is one 32-bit buffer range: 3*D*D*2 >= 2^31


def attn(**kw):
    a = dict(q=A, k=A, v=A, nq=16, nkv=64, heads=2, hd=64, scale=0.0, out=A, rows=None, nout=0, lse=None,
             ws=None, ws_bytes=0)
    a.update(kw)
    return lib().tsa_sparse_query_attention(a["q"], a["k"], a["v"], a["nq"], a["nkv"], a["heads"],
                                            a["hd"], a["scale"], a["out"], a["rows"], a["nout"],
                                            a["lse"], a["ws"], a["ws_bytes"], None)


def test_attention_validation():
    assert attn(nq=0) == B.OK
    assert attn(q=None) == B.ERR_INVALID_ARG
    assert attn(out=None) == B.ERR_INVALID_ARG
    assert attn(hd=96) == B.ERR_SHAPE
    assert attn(heads=0) == B.ERR_SHAPE
    assert attn(nkv=0) == B.ERR_SHAPE
    assert attn(nq=-3) == B.ERR_SHAPE
    assert attn(scale=float("inf")) == B.ERR_INVALID_ARG
    assert attn(k=U) == B.ERR_ALIGNMENT
    assert attn(lse=A + 2) == B.ERR_ALIGNMENT
    # caches of 2 GiB and more are accepted (buffer ranges rebased per key tile); n_q = 0 launches nothing
    assert attn(nkv=1 << 20, heads=8, hd=128, nq=0) == B.OK
    assert attn(nkv=(1 << 31) - 1, heads=64, hd=128, nq=0) == B.OK
    assert attn(nkv=1 << 31, heads=8, hd=128, nq=0) == B.ERR_SHAPE  # rows past 2^31 - 1
    assert attn(ws=U, ws_bytes=1 << 20) == B.ERR_ALIGNMENT
    assert attn(nq=0, ws=A, ws_bytes=0) == B.OK
    f = lib()
    assert f.tsa_attention_workspace_bytes(0, 64, 2, 64) == 0
    assert f.tsa_attention_workspace_bytes(16, 64, 2, 96) == 0
    assert f.tsa_attention_workspace_bytes(16, 64, 0, 128) == 0
    assert f.tsa_attention_workspace_bytes(16, 0, 2, 128) == 0


def test_row_mover_validation():
    f = lib()
    assert f.tsa_kv_cache_sync(A, A, A, 0, A, A, 64, 64, None) == B.OK
    assert f.tsa_kv_cache_sync(None, A, A, 4, A, A, 64, 64, None) == B.ERR_INVALID_ARG
    assert f.tsa_kv_cache_sync(A, A, A, 65, A, A, 64, 64, None) == B.ERR_SHAPE
    assert f.tsa_kv_cache_sync(A, A, A, 4, A, A, 64, 60, None) == B.ERR_SHAPE
    assert f.tsa_kv_cache_sync(A, U, A, 4, A, A, 64, 64, None) == B.ERR_ALIGNMENT
    assert f.tsa_scatter_out(A, A, 0, A, 64, 64, None) == B.OK
    assert f.tsa_scatter_out(A, None, 4, A, 64, 64, None) == B.ERR_INVALID_ARG
    assert f.tsa_scatter_out(A, A, 70, A, 64, 64, None) == B.ERR_SHAPE
    assert f.tsa_gather_rows(A, 64, A, 0, 64, None, 0, 0.0, A, None) == B.OK
    assert f.tsa_gather_rows(A, 64, A, 4, 64, None, 0, 0.0, U, None) == B.ERR_ALIGNMENT
    assert f.tsa_gather_rows(None, 64, A, 4, 64, None, 0, 0.0, A, None) == B.ERR_INVALID_ARG


def test_assign_groups_validation():
    f = lib()
    counts = (ctypes.c_int64 * 3)(16, 16, 32)
    periods = (ctypes.c_uint8 * 3)(1, 2, 4)
    cp, pp = ctypes.cast(counts, ctypes.c_void_p), ctypes.cast(periods, ctypes.c_void_p)
    assert f.tsa_assign_groups(A, 64, 3, cp, pp, A, None, 0, None) == B.ERR_WORKSPACE
    assert f.tsa_assign_groups(A, 65, 3, cp, pp, A, A, 1024, None) == B.ERR_SHAPE
    assert f.tsa_assign_groups(A, 64, 0, cp, pp, A, A, 1024, None) == B.ERR_SHAPE
    assert f.tsa_assign_groups(U, 64, 3, cp, pp, A, A, 1024, None) == B.ERR_ALIGNMENT
    assert f.tsa_assign_groups(None, 64, 3, cp, pp, A, A, 1024, None) == B.ERR_INVALID_ARG
    assert f.tsa_assign_groups(A, 0, 1, cp, pp, A, None, 0, None) == B.ERR_SHAPE  # counts sum 16 != 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(B, "_lib_handle", None)
    with pytest.raises(ImportError):
        B.lib()


def test_rope_and_causal_validation():
    f = lib()

    def qr(**kw):
        a = dict(x=A, dt=B.BF16, nx=64, rows=None, n=16, dim=128, w=A, q=A, k=A, v=A, cache=0, nc=0,
                 eps=None, off=0, sigma=0.0, heads=2, h=4, w_=4, base=10000.0)
        a.update(kw)
        return f.tsa_qkv_active_rope(a["x"], a["dt"], a["nx"], a["rows"], a["n"], a["dim"], a["w"], a["q"],
                                     a["k"], a["v"], a["cache"], a["nc"], a["eps"], a["off"], a["sigma"],
                                     a["heads"], a["h"], a["w_"], a["base"], None)
    assert qr(n=0) == B.OK
    assert qr(heads=3) == B.ERR_SHAPE       # 128 / 3 not an integer head dim
    assert qr(heads=64) == B.ERR_SHAPE      # head dim 2 < 6
    assert qr(h=0) == B.ERR_SHAPE
    assert qr(base=0.0) == B.ERR_INVALID_ARG
    assert qr(base=float("inf")) == B.ERR_INVALID_ARG
    assert qr(x=None) == B.ERR_INVALID_ARG
    assert qr(w=U) == B.ERR_ALIGNMENT

    def fc(**kw):
        a = dict(q=A, k=A, v=A, nq=16, nkv=64, heads=2, hd=64, scale=0.0, qt=A, ft=8, out=A, rows=None, nout=0,
                 lse=None)
        a.update(kw)
        return f.tsa_frame_causal_attention(a["q"], a["k"], a["v"], a["nq"], a["nkv"], a["heads"], a["hd"],
                                            a["scale"], a["qt"], a["ft"], a["out"], a["rows"], a["nout"],
                                            a["lse"], None)
    assert fc(nq=0) == B.OK
    assert fc(qt=None) == B.ERR_INVALID_ARG
    assert fc(ft=0) == B.ERR_SHAPE
    assert fc(hd=96) == B.ERR_SHAPE
    assert fc(qt=A + 2) == B.ERR_ALIGNMENT


def test_reuse_validation():
    f = lib()
    assert tsa.reuse_workspace_bytes(100, 3) == 2 * 100 * 3 * 3 * 4
    assert tsa.reuse_workspace_bytes(0, 3) == 0
    big = 1 << 40

    def ru(th=(0.1, 0.1, 0.1), **kw):
        t = (ctypes.c_float * 3)(*th)
        a = dict(v=A, n=64, heads=2, hd=128, h=4, w=4, eff=A + big, src=None, delta=None, ws=A + 2 * big,
                 wsb=2 * 64 * 2 * 3 * 4)
        a.update(kw)
        return f.tsa_timeripple_reuse(a["v"], a["n"], a["heads"], a["hd"], a["h"], a["w"],
                                      ctypes.cast(t, ctypes.c_void_p), a["eff"], a["src"], a["delta"], a["ws"],
                                      a["wsb"], None)
    assert ru(n=0) == B.OK
    assert ru(n=0, ws=None, wsb=0) == B.OK
    assert ru(v=None) == B.ERR_INVALID_ARG
    assert ru(eff=None) == B.ERR_INVALID_ARG
    assert ru(th=(0.1, float("nan"), 0.1)) == B.ERR_INVALID_ARG
    assert ru(th=(-0.1, 0.1, 0.1)) == B.ERR_INVALID_ARG
    assert ru(eff=A + 64) == B.ERR_INVALID_ARG  # overlaps v
    assert ru(hd=96) == B.ERR_SHAPE
    assert ru(heads=0) == B.ERR_SHAPE
    assert ru(h=0) == B.ERR_SHAPE
    assert ru(v=U) == B.ERR_ALIGNMENT
    assert ru(src=A + 2) == B.ERR_ALIGNMENT
    assert ru(ws=None) == B.ERR_WORKSPACE
    assert ru(wsb=100) == B.ERR_WORKSPACE

    # the variant without a workspace: the same checks, and at most 2^20 token-heads
    def rn(th=(0.1, 0.1, 0.1), **kw):
        t = (ctypes.c_float * 3)(*th)
        a = dict(v=A, n=64, heads=2, hd=128, h=4, w=4, eff=A + big, src=None, delta=None)
        a.update(kw)
        return f.tsa_timeripple_reuse_noalloc(a["v"], a["n"], a["heads"], a["hd"], a["h"], a["w"],
                                              ctypes.cast(t, ctypes.c_void_p), a["eff"], a["src"], a["delta"],
                                              None)
    assert tsa.reuse_noalloc_max_token_heads() == 1 << 20
    assert rn(n=0) == B.OK
    assert rn(v=None) == B.ERR_INVALID_ARG
    assert rn(th=(0.1, float("nan"), 0.1)) == B.ERR_INVALID_ARG
    assert rn(eff=A + 64) == B.ERR_INVALID_ARG
    assert rn(hd=96) == B.ERR_SHAPE
    assert rn(v=U) == B.ERR_ALIGNMENT
    assert rn(n=(1 << 19) + 1, heads=2) == B.ERR_SHAPE  # above 2^20 token-heads


def test_qkv_rows_to_cache_validation():
    f = lib()

    def rc(**kw):
        a = dict(a=A, n=16, dim=128, rows=A, w=A, q=None, k=A, v=A, nc=64, heads=0, h=1, w_=1, base=10000.0)
        a.update(kw)
        return f.tsa_qkv_rows_to_cache(a["a"], a["n"], a["dim"], a["rows"], a["w"], a["q"], a["k"], a["v"],
                                       a["nc"], a["heads"], a["h"], a["w_"], a["base"], None)
    assert rc(n=0) == B.OK
    assert rc(rows=None) == B.ERR_INVALID_ARG
    assert rc(a=None) == B.ERR_INVALID_ARG
    assert rc(dim=96) == B.ERR_SHAPE
    assert rc(heads=3) == B.ERR_SHAPE
    assert rc(heads=2, h=0) == B.ERR_SHAPE
    assert rc(heads=2, h=4, w_=4, base=0.0) == B.ERR_INVALID_ARG
    assert rc(a=U) == B.ERR_ALIGNMENT
    assert rc(rows=A + 2) == B.ERR_ALIGNMENT
    assert rc(dim=19008) == B.ERR_SHAPE  # 3*D*D*2 >= 2^31
