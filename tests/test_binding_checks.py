"""The Python binding checks every tensor argument's dtype and extent before calling the
C ABI (which sees only pointers): a tensor too small for what a call touches raises
ValueError on the host instead of being read or written past its end on the GPU.  CPU
tensors are used here; a well-formed call then stops at the device check."""

from __future__ import annotations

import pytest
import torch

from token_sparse_attention_rel_amd import _binding as B

bf, f32, i32, u8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8


def T(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_well_formed_call_stops_at_device_check():
    raises("live on the GPU", B.kv_cache_sync, T(4, 64), T(4, 64), T(4, dtype=i32), 4, T(10, 64), T(10, 64))


def test_kv_cache_sync_extents():
    raises("k_a: 3 rows", B.kv_cache_sync, T(3, 64), T(4, 64), T(4, dtype=i32), 4, T(10, 64), T(10, 64))
    raises("v_cache: 9 rows", B.kv_cache_sync, T(4, 64), T(4, 64), T(4, dtype=i32), 4, T(10, 64), T(9, 64))
    raises("rows: 3 elements", B.kv_cache_sync, T(4, 64), T(4, 64), T(3, dtype=i32), 4, T(10, 64), T(10, 64))
    raises("rows: dtype", B.kv_cache_sync, T(4, 64), T(4, 64), T(4, dtype=torch.int64), 4, T(10, 64), T(10, 64))
    raises("k_a: shape", B.kv_cache_sync, T(4, 32), T(4, 64), T(4, dtype=i32), 4, T(10, 64), T(10, 64))


def test_qkv_extents():
    x, w = T(10, 64), T(192, 64)
    raises("w_qkv: 191 rows", B.qkv_active, x, T(4, dtype=i32), 4, T(191, 64), k_out=T(4, 64), v_out=T(4, 64))
    raises("q_out: 3 rows", B.qkv_active, x, T(4, dtype=i32), 4, w, q_out=T(3, 64), k_out=T(4, 64),
           v_out=T(4, 64))
    raises("n_cache = 12 exceeds", B.qkv_active, x, T(4, dtype=i32), 4, w, k_out=T(10, 64), v_out=T(10, 64),
           out_is_cache=True, n_cache=12)
    raises("rows is None but n = 11", B.qkv_active, x, None, 11, w, k_out=T(11, 64), v_out=T(11, 64))
    raises("eps: 9 rows", B.qkv_active, x, T(4, dtype=i32), 4, w, k_out=T(4, 64), v_out=T(4, 64),
           eps=T(9, 64), sigma=0.5)
    raises("k_out: dtype", B.qkv_active, x, T(4, dtype=i32), 4, w, k_out=T(4, 64, dtype=f32), v_out=T(4, 64))


def test_attention_extents():
    q, k, v = T(5, 256), T(40, 256), T(40, 256)
    raises("q: 4 rows", B.sparse_query_attention, T(4, 256), k, v, 5, 2, 128, T(5, 256))
    raises("out: 4 rows", B.sparse_query_attention, q, k, v, 5, 2, 128, T(4, 256))
    raises("v_cache: 39 rows", B.sparse_query_attention, q, k, T(39, 256), 5, 2, 128, T(5, 256))
    raises("lse_out: 9 elements", B.sparse_query_attention, q, k, v, 5, 2, 128, T(5, 256), lse_out=T(9, dtype=f32))
    raises("out_rows: 4 elements", B.sparse_query_attention, q, k, v, 5, 2, 128, T(40, 256),
           out_rows=T(4, dtype=i32))
    raises("q_tokens: 4 elements", B.frame_causal_attention, q, k, v, 5, 2, 128, T(4, dtype=i32), 8, T(5, 256))
    raises("k_cache: shape", B.sparse_query_attention, q, T(40, 128), v, 5, 2, 128, T(5, 256))


def test_select_and_scores_extents():
    x = T(100, 64)
    kw = dict(mask_out=T(100, dtype=u8), idx_out=T(100, dtype=i32), n_active_out=T(1, dtype=i32))
    raises("idx_out: 99", B.select_active, x, x, 0, B.SELECT_TOPK, k=10, **{**kw, "idx_out": T(99, dtype=i32)})
    raises("x_ref: 99 rows", B.select_active, x, T(99, 64), 0, B.SELECT_TOPK, k=10, **kw)
    raises("x_ref must have the dtype", B.select_active, x, T(100, 64, dtype=f32), 0, B.SELECT_TOPK, k=10, **kw)
    raises("aux_in: 99", B.select_active, None, None, 0, B.SELECT_MASK, aux_in=T(99, dtype=u8), n_rows=100, **kw)
    raises("n_rows is required", B.select_active, None, None, 0, B.SELECT_MASK, aux_in=T(100, dtype=u8), **kw)
    raises("scores_out: 99", B.token_scores, x, x, T(99, dtype=f32))


def test_row_movers_frames_and_reuse_extents():
    raises("dst: 3 rows", B.gather_rows, T(10, 64), T(4, dtype=i32), 4, T(3, 64))
    raises("o_a: 3 rows", B.scatter_out, T(3, 64), T(4, dtype=i32), 4, T(10, 64))
    raises("v_hat: 9 rows", B.euler_update, T(10, 64, dtype=f32), T(9, 64), 0.1)
    raises("x: 11 rows", B.lif_mask, T(11, 64), 3, 4, 0.1, 0.1, T(12, dtype=u8))
    raises("mask_out: 11", B.lif_mask, T(12, 64), 3, 4, 0.1, 0.1, T(11, dtype=u8))
    raises("mask: 11", B.restore_frames, T(12, 64), T(11, dtype=u8), 3, 4)
    raises("eff_out: 11 rows", B.timeripple_reuse, T(12, 256), 2, 128, 3, 4, (0.1, 0.1, 0.1), T(11, 256), None)
    raises("src_out: 71", B.timeripple_reuse, T(12, 256), 2, 128, 3, 4, (0.1, 0.1, 0.1), T(12, 256), None,
           src_out=T(71, dtype=i32))
    raises("a: 3 rows", B.qkv_rows_to_cache, T(3, 64), T(4, dtype=i32), 4, T(192, 64), T(10, 64), T(10, 64))
