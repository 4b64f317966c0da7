"""The debug build (libtsa_debug.so, TSA_DEBUG) checks every index list before a kernel
reads it: out-of-range, negative, repeated or descending entries come back as
TSA_ERR_SHAPE and nothing is written; valid lists give the release build's bits."""

from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest
import torch

import gpu_util as G

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                         "token_sparse_attention_rel_amd", "libtsa_debug.so")
OK, ERR_SHAPE = 0, 2


@pytest.fixture(scope="module")
def dbg():
    G.need_gpu()
    from token_sparse_attention_rel_amd import _binding as B
    if not os.path.exists(DEBUG_LIB):
        raise FileNotFoundError(f"{DEBUG_LIB} is missing: python -m token_sparse_attention_rel_amd.build --debug")
    h = ctypes.CDLL(DEBUG_LIB)
    for name, (res, args) in B._SIGNATURES.items():
        fn = getattr(h, name)
        fn.restype = res
        fn.argtypes = args
    return h


def p(t):
    return None if t is None else t.data_ptr()


def idx(vals):
    return torch.tensor(vals, dtype=torch.int32, device="cuda")


BAD_LISTS = {"descending": [5, 3, 9], "repeated": [3, 3, 9], "negative": [-1, 3, 9], "past_end": [3, 9, 100]}


def test_row_movers_reject_bad_lists(dbg):
    n_cache, dim = 100, 64
    src = torch.randn(3, dim, device="cuda").to(torch.bfloat16)
    for what in ("cache_sync", "scatter", "gather"):
        for name, vals in list(BAD_LISTS.items()) + [("valid", [3, 9, 99])]:
            kc = torch.full((n_cache, dim), 2.0, dtype=torch.bfloat16, device="cuda")
            vc = kc.clone()
            rows = idx(vals)
            if what == "cache_sync":
                st = dbg.tsa_kv_cache_sync(p(src), p(src), p(rows), 3, p(kc), p(vc), n_cache, dim, None)
            elif what == "scatter":
                st = dbg.tsa_scatter_out(p(src), p(rows), 3, p(kc), n_cache, dim, None)
            else:
                dst = torch.full((3, dim), 2.0, dtype=torch.bfloat16, device="cuda")
                st = dbg.tsa_gather_rows(p(kc), n_cache, p(rows), 3, dim, None, 0, 0.0, p(dst), None)
            torch.cuda.synchronize()
            print(f"  {what} {name}: status {st}", flush=True)
            if name == "valid":
                assert st == OK
                if what != "gather":
                    assert torch.equal(kc[rows.long()], src)
                else:
                    assert bool((dst == 2.0).all())
            else:
                assert st == ERR_SHAPE
                assert bool((kc == 2.0).all()) and bool((vc == 2.0).all())


def test_projection_rejects_bad_lists(dbg):
    n_x, dim = 50, 128
    x = torch.randn(n_x, dim, device="cuda").to(torch.bfloat16)
    w = (torch.randn(3 * dim, dim, device="cuda") / dim ** 0.5).to(torch.bfloat16)
    for name, vals in list(BAD_LISTS.items()) + [("past_x_rows", [3, 9, 50]), ("valid", [3, 9, 49])]:
        rows = idx(vals)
        kc = torch.full((120, dim), 2.0, dtype=torch.bfloat16, device="cuda")
        vc = kc.clone()
        q = torch.full((3, dim), 2.0, dtype=torch.bfloat16, device="cuda")
        st = dbg.tsa_qkv_active(p(x), 1, n_x, p(rows), 3, dim, p(w), p(q), p(kc), p(vc), 1, 120, None, 0, 0.0, None)
        st2 = dbg.tsa_qkv_rows_to_cache(p(x), 3, dim, p(rows), p(w), None, p(kc), p(vc), 40, 0, 1, 1, 10000.0, None)
        torch.cuda.synchronize()
        print(f"  qkv {name}: status {st}, rows_to_cache (40 cache rows) {st2}", flush=True)
        if name == "valid":
            assert st == OK and st2 == ERR_SHAPE  # 49 is past the 40 cache rows of the second call
        elif name == "past_x_rows":
            assert st == ERR_SHAPE and st2 == ERR_SHAPE
        else:
            assert st == ERR_SHAPE and st2 == ERR_SHAPE
            assert bool((q == 2.0).all()) and bool((kc == 2.0).all())


def test_attention_out_rows_and_query_tokens(dbg):
    import token_sparse_attention_rel_amd as t
    heads, hd, n_kv, n_q, n_out = 2, 64, 300, 3, 400
    q = torch.randn(n_q, heads * hd, device="cuda").to(torch.bfloat16)
    k = torch.randn(n_kv, heads * hd, device="cuda").to(torch.bfloat16)
    v = torch.randn(n_kv, heads * hd, device="cuda").to(torch.bfloat16)
    bad = {k: v for k, v in BAD_LISTS.items() if k != "past_end"}  # 100 is a valid row of 400
    for name, vals in list(bad.items()) + [("past_n_out", [3, 9, 400]), ("valid", [3, 9, 399])]:
        rows = idx(vals)
        out = torch.full((n_out, heads * hd), 2.0, dtype=torch.bfloat16, device="cuda")
        st = dbg.tsa_sparse_query_attention(p(q), p(k), p(v), n_q, n_kv, heads, hd, 0.0, p(out), p(rows), n_out,
                                            None, None, 0, None)
        torch.cuda.synchronize()
        print(f"  attention out_rows {name}: status {st}", flush=True)
        if name == "valid":
            assert st == OK
            ref_out = torch.full_like(out, 2.0)
            t.sparse_query_attention(q, k, v, n_q, heads, hd, ref_out, out_rows=rows)
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out)  # the release build's bits
        else:
            assert st == ERR_SHAPE and bool((out == 2.0).all())
    toks = idx([5, -2, 7])
    out = torch.full((n_out, heads * hd), 2.0, dtype=torch.bfloat16, device="cuda")
    st = dbg.tsa_frame_causal_attention(p(q), p(k), p(v), n_q, n_kv, heads, hd, 0.0, p(toks), 100, p(out),
                                        p(idx([3, 9, 399])), n_out, None, None)
    torch.cuda.synchronize()
    assert st == ERR_SHAPE and bool((out == 2.0).all())
