"""ctypes binding of libtsa.so: argument marshalling only.

Each function here has the name of a C entry point without its ``tsa_``
prefix and forwards to it unchanged; all computation happens in the HIP
kernels behind the C ABI.  Tensors are passed as device pointers (their
``data_ptr()``); PyTorch only provides the memory and the stream.  A nonzero
status raises :class:`TsaError`.

There is no fallback: if the library is missing, loading it raises.
"""

from __future__ import annotations

import ctypes
import os

# The in-tree build; TSA_LIB names another build of the same library (the debug build with
# index-list checks, or a sanitizer build of the host code).
_LIB_PATH = os.environ.get("TSA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsa.so")

# Values of the C enums (include/tsa.h).
OK = 0
ERR_INVALID_ARG, ERR_SHAPE, ERR_DTYPE, ERR_ALIGNMENT, ERR_WORKSPACE, ERR_HIP = 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1
SCORE_REL_L1, SCORE_ABS_L1 = 0, 1
SELECT_TOPK, SELECT_THRESHOLD, SELECT_MASK, SELECT_SCHEDULE = 0, 1, 2, 3

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_f32 = ctypes.c_float
_size = ctypes.c_size_t

_SIGNATURES = {
    "tsa_abi_version": (_int, []),
    "tsa_status_string": (ctypes.c_char_p, [_int]),
    "tsa_select_workspace_bytes": (_size, [_i64]),
    "tsa_select_active": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _int, _int, _i64, _f32, _vp, _i64,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _size, _vp]),
    "tsa_assign_groups": (_int, [_vp, _i64, _int, _vp, _vp, _vp, _vp, _size, _vp]),
    "tsa_qkv_active": (_int, [_vp, _int, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _int, _i64,
                              _vp, _i64, _f32, _vp]),
    "tsa_kv_cache_sync": (_int, [_vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _vp]),
    "tsa_sparse_query_attention": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _f32, _vp, _vp,
                                          _i64, _vp, _vp, _size, _vp]),
    "tsa_attention_workspace_bytes": (_size, [_i64, _i64, _int, _int]),
    "tsa_scatter_out": (_int, [_vp, _vp, _i64, _vp, _i64, _i64, _vp]),
    "tsa_gather_rows": (_int, [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _f32, _vp, _vp]),
    "tsa_qkv_active_rope": (_int, [_vp, _int, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _int, _i64,
                                   _vp, _i64, _f32, _int, _i64, _i64, _f32, _vp]),
    "tsa_frame_causal_attention": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _f32, _vp, _i64, _vp, _vp,
                                          _i64, _vp, _vp]),
    "tsa_token_scores": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _vp]),
    "tsa_euler_update": (_int, [_vp, _int, _vp, _i64, _i64, _f32, _vp]),
    "tsa_lif_mask": (_int, [_vp, _int, _i64, _i64, _i64, _int, _f32, _f32, _vp, _vp, _vp, _vp]),
    "tsa_restore_frames": (_int, [_vp, _int, _vp, _i64, _i64, _i64, _vp]),
    "tsa_reuse_workspace_bytes": (_size, [_i64, _int]),
    "tsa_qkv_rows_to_cache": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _int, _i64, _i64, _f32, _vp]),
    "tsa_timeripple_reuse": (_int, [_vp, _i64, _int, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _size, _vp]),
    "tsa_timeripple_reuse_noalloc": (_int, [_vp, _i64, _int, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "tsa_reuse_noalloc_max_token_heads": (_size, []),
}

_lib_handle = None


class TsaError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libtsa.so with argument/return types set (raises if it is not built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is missing: build it with `python -m token_sparse_attention_rel_amd.build`"
            )
        h = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = h
    return _lib_handle


def lib_path() -> str:
    return _LIB_PATH


def status_string(status: int) -> str:
    return lib().tsa_status_string(int(status)).decode()


def abi_version() -> int:
    return lib().tsa_abi_version()


def select_workspace_bytes(n_rows: int) -> int:
    return lib().tsa_select_workspace_bytes(int(n_rows))


# ------------------------------------------------------------- marshalling

def _ptr(t):
    """Device pointer of a tensor (None -> NULL; ints pass through as raw addresses)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(name: str, status: int) -> None:
    if status != OK:
        raise TsaError(name, status)


_DTYPES = {"bf16": "bfloat16", "f32": "float32", "i32": "int32", "u8": "uint8"}


def _need(t, name, dtypes, *, rows=None, cols=None, numel=None):
    """Check a tensor argument before the call (None passes: the C ABI rejects a missing
    required buffer itself): one of ``dtypes``, and room for what the call touches -- at
    least ``rows`` rows of exactly ``cols`` columns (2-D), or at least ``numel`` elements.
    The C ABI receives bare pointers and cannot see their extents; a tensor that is too
    small would otherwise be read or written past its end on the GPU."""
    if t is None:
        return
    if str(t.dtype).replace("torch.", "") not in tuple(_DTYPES[d] for d in dtypes):
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(dtypes)}")
    if cols is not None and (t.dim() != 2 or t.shape[1] != cols):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected [rows, {cols}]")
    if rows is not None and (t.dim() == 0 or t.shape[0] < rows):
        raise ValueError(f"{name}: {t.shape[0] if t.dim() else 0} rows, at least {rows} needed")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {numel} needed")


def _rows_index(rows, n, n_src, name="rows"):
    """Row list of n entries, or None (identity: then n rows must exist)."""
    if rows is None:
        if n > n_src:
            raise ValueError(f"{name} is None but n = {n} exceeds the {n_src} rows available")
    else:
        _need(rows, name, ("i32",), numel=n)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# --------------------------------------------------------------- entry points

def select_active(x_cur, x_ref, ref_row_offset, mode, *, k=0, tau=0.0, aux_in=None, step=0,
                  score_kind=SCORE_REL_L1, scores_out=None, mask_out, idx_out, pidx_out=None,
                  n_active_out, workspace=None, stream=None, n_rows=None, dim=None):
    """a1-a3 (tsa_select_active).  x_cur/x_ref are [N, D] fp32 or bf16 device tensors."""
    if x_cur is not None:
        n_rows = x_cur.shape[0] if n_rows is None else n_rows
        dim = x_cur.shape[1] if dim is None else dim
        dt = _dtype_code(x_cur)
        _need(x_cur, "x_cur", ("bf16", "f32"), rows=n_rows, cols=dim)
        if x_ref is not None and x_ref.dtype != x_cur.dtype:
            raise ValueError("x_ref must have the dtype of x_cur")
        _need(x_ref, "x_ref", ("bf16", "f32"), rows=n_rows, cols=dim)
    else:
        dt = BF16
        dim = 0 if dim is None else dim
    if n_rows is None:
        raise ValueError("n_rows is required without x_cur")
    _need(aux_in, "aux_in", ("u8",), numel=n_rows)
    _need(scores_out, "scores_out", ("f32",), numel=n_rows)
    _need(mask_out, "mask_out", ("u8",), numel=n_rows)
    _need(idx_out, "idx_out", ("i32",), numel=n_rows)
    _need(pidx_out, "pidx_out", ("i32",), numel=n_rows)
    _need(n_active_out, "n_active_out", ("i32",), numel=1)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().tsa_select_active(
        _ptr(x_cur), _ptr(x_ref), int(ref_row_offset), int(n_rows), int(dim), dt, int(score_kind),
        int(mode), int(k), float(tau), _ptr(aux_in), int(step), _ptr(scores_out), _ptr(mask_out),
        _ptr(idx_out), _ptr(pidx_out), _ptr(n_active_out), _ptr(workspace), ws_bytes, _stream(stream))
    _check("tsa_select_active", st)


def assign_groups(scores, group_counts, group_periods, period_out, workspace, stream=None):
    """HSA rank groups (tsa_assign_groups); counts/periods are host sequences."""
    n = scores.shape[0]
    _need(scores, "scores", ("f32",), numel=n)
    _need(period_out, "period_out", ("u8",), numel=n)
    g = len(group_counts)
    counts = (ctypes.c_int64 * g)(*[int(c) for c in group_counts])
    periods = (ctypes.c_uint8 * g)(*[int(p) for p in group_periods])
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().tsa_assign_groups(_ptr(scores), int(n), g, ctypes.cast(counts, _vp),
                                 ctypes.cast(periods, _vp), _ptr(period_out), _ptr(workspace),
                                 ws_bytes, _stream(stream))
    _check("tsa_assign_groups", st)


def qkv_active(x, rows, n, w_qkv, *, q_out=None, k_out, v_out, out_is_cache=False, n_cache=0,
               eps=None, src_row_offset=0, sigma=0.0, stream=None):
    """a4-a5 (+a6 when out_is_cache) (tsa_qkv_active)."""
    dim = x.shape[1]
    _need(x, "x", ("bf16", "f32"), cols=dim)
    _rows_index(rows, n, x.shape[0])
    _need(w_qkv, "w_qkv", ("bf16",), rows=3 * dim, cols=dim)
    _need(q_out, "q_out", ("bf16",), rows=n, cols=dim)
    if out_is_cache and k_out is not None and n_cache > k_out.shape[0]:
        raise ValueError(f"n_cache = {n_cache} exceeds the {k_out.shape[0]} rows of k_out")
    _need(k_out, "k_out", ("bf16",), rows=n_cache if out_is_cache else n, cols=dim)
    _need(v_out, "v_out", ("bf16",), rows=n_cache if out_is_cache else n, cols=dim)
    _need(eps, "eps", ("bf16",), rows=x.shape[0], cols=dim)
    st = lib().tsa_qkv_active(
        _ptr(x), _dtype_code(x), int(x.shape[0]), _ptr(rows), int(n), int(x.shape[1]), _ptr(w_qkv),
        _ptr(q_out), _ptr(k_out), _ptr(v_out), 1 if out_is_cache else 0, int(n_cache), _ptr(eps),
        int(src_row_offset), float(sigma), _stream(stream))
    _check("tsa_qkv_active", st)


def kv_cache_sync(k_a, v_a, rows, n, k_cache, v_cache, stream=None):
    """a6 (tsa_kv_cache_sync)."""
    dim = k_cache.shape[1]
    _need(k_cache, "k_cache", ("bf16",), cols=dim)
    _need(v_cache, "v_cache", ("bf16",), rows=k_cache.shape[0], cols=dim)
    _need(k_a, "k_a", ("bf16",), rows=n, cols=dim)
    _need(v_a, "v_a", ("bf16",), rows=n, cols=dim)
    _need(rows, "rows", ("i32",), numel=n)
    st = lib().tsa_kv_cache_sync(_ptr(k_a), _ptr(v_a), _ptr(rows), int(n), _ptr(k_cache),
                                 _ptr(v_cache), int(k_cache.shape[0]), int(k_cache.shape[1]),
                                 _stream(stream))
    _check("tsa_kv_cache_sync", st)


def attention_workspace_bytes(n_q, n_kv, heads, head_dim):
    """tsa_attention_workspace_bytes (current device)."""
    return int(lib().tsa_attention_workspace_bytes(int(n_q), int(n_kv), int(heads), int(head_dim)))


def sparse_query_attention(q, k_cache, v_cache, n_q, heads, head_dim, out, *, out_rows=None,
                           scale=0.0, lse_out=None, workspace=None, stream=None):
    """a7 (+a8 when out_rows is given) (tsa_sparse_query_attention).  ``workspace``:
    a device tensor of at least attention_workspace_bytes() bytes, or None."""
    dim = int(heads) * int(head_dim)
    _need(k_cache, "k_cache", ("bf16",), cols=dim)
    _need(v_cache, "v_cache", ("bf16",), rows=k_cache.shape[0], cols=dim)
    _need(q, "q", ("bf16",), rows=n_q, cols=dim)
    _need(out, "out", ("bf16",), rows=0 if out_rows is not None else n_q, cols=dim)
    _need(out_rows, "out_rows", ("i32",), numel=n_q)
    _need(lse_out, "lse_out", ("f32",), numel=int(heads) * int(n_q))
    n_out = out.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().tsa_sparse_query_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), int(n_q), int(k_cache.shape[0]), int(heads),
        int(head_dim), float(scale), _ptr(out), _ptr(out_rows), int(n_out), _ptr(lse_out),
        _ptr(workspace), ws_bytes, _stream(stream))
    _check("tsa_sparse_query_attention", st)


def scatter_out(o_a, rows, n, out, stream=None):
    """a8 (tsa_scatter_out)."""
    dim = out.shape[1]
    _need(out, "out", ("bf16",), cols=dim)
    _need(o_a, "o_a", ("bf16",), rows=n, cols=dim)
    _need(rows, "rows", ("i32",), numel=n)
    st = lib().tsa_scatter_out(_ptr(o_a), _ptr(rows), int(n), _ptr(out), int(out.shape[0]),
                               int(out.shape[1]), _stream(stream))
    _check("tsa_scatter_out", st)


def gather_rows(x, rows, n, dst, *, eps=None, src_row_offset=0, sigma=0.0, stream=None):
    """a4 alone (tsa_gather_rows)."""
    dim = x.shape[1]
    _need(x, "x", ("bf16",), cols=dim)
    _rows_index(rows, n, x.shape[0])
    _need(dst, "dst", ("bf16",), rows=n, cols=dim)
    _need(eps, "eps", ("bf16",), rows=x.shape[0], cols=dim)
    st = lib().tsa_gather_rows(_ptr(x), int(x.shape[0]), _ptr(rows), int(n), int(x.shape[1]),
                               _ptr(eps), int(src_row_offset), float(sigma), _ptr(dst),
                               _stream(stream))
    _check("tsa_gather_rows", st)


def euler_update(x, v_hat, dt, stream=None):
    """Cached Euler update x <- x + dt * v_hat over all rows (tsa_euler_update)."""
    _need(x, "x", ("f32", "bf16"), cols=x.shape[1] if x.dim() == 2 else -1)
    _need(v_hat, "v_hat", ("bf16",), rows=x.shape[0], cols=x.shape[1])
    st = lib().tsa_euler_update(_ptr(x), _dtype_code(x), _ptr(v_hat), int(x.shape[0]), int(x.shape[1]),
                                float(dt), _stream(stream))
    _check("tsa_euler_update", st)


def lif_mask(x, frames, hw, tau_short, tau_long, mask_out, *, score_kind=SCORE_ABS_L1, short_out=None,
             long_out=None, stream=None):
    """Long/short-term inter-frame pruning mask (tsa_lif_mask); x is [frames*hw, dim]."""
    n = int(frames) * int(hw)
    _need(x, "x", ("bf16", "f32"), rows=n, cols=x.shape[1] if x.dim() == 2 else -1)
    _need(mask_out, "mask_out", ("u8",), numel=n)
    _need(short_out, "short_out", ("f32",), numel=n)
    _need(long_out, "long_out", ("f32",), numel=n)
    st = lib().tsa_lif_mask(_ptr(x), _dtype_code(x), int(frames), int(hw), int(x.shape[1]), int(score_kind),
                            float(tau_short), float(tau_long), _ptr(mask_out), _ptr(short_out),
                            _ptr(long_out), _stream(stream))
    _check("tsa_lif_mask", st)


def restore_frames(buf, mask, frames, hw, stream=None):
    """Forward fill of pruned tokens from the previous frame (tsa_restore_frames)."""
    n = int(frames) * int(hw)
    _need(buf, "buf", ("bf16", "f32"), rows=n, cols=buf.shape[1] if buf.dim() == 2 else -1)
    _need(mask, "mask", ("u8",), numel=n)
    st = lib().tsa_restore_frames(_ptr(buf), _dtype_code(buf), _ptr(mask), int(frames), int(hw),
                                  int(buf.shape[1]), _stream(stream))
    _check("tsa_restore_frames", st)


def qkv_rows_to_cache(a, rows, n, w_qkv, k_cache, v_cache, *, q_out=None, rope=None, heads=0, stream=None):
    """K/V (and Q) of compact rows a[r], written to cache rows rows[r] (tsa_qkv_rows_to_cache);
    rope = (height, width, base) with heads > 0 rotates Q and K by the tokens' positions."""
    h, w, base = rope if rope is not None else (1, 1, 10000.0)
    dim = a.shape[1]
    _need(a, "a", ("bf16",), rows=n, cols=dim)
    _need(rows, "rows", ("i32",), numel=n)
    _need(w_qkv, "w_qkv", ("bf16",), rows=3 * dim, cols=dim)
    _need(k_cache, "k_cache", ("bf16",), cols=dim)
    _need(v_cache, "v_cache", ("bf16",), rows=k_cache.shape[0], cols=dim)
    _need(q_out, "q_out", ("bf16",), rows=n, cols=dim)
    st = lib().tsa_qkv_rows_to_cache(_ptr(a), int(n), int(a.shape[1]), _ptr(rows), _ptr(w_qkv), _ptr(q_out),
                                      _ptr(k_cache), _ptr(v_cache), int(k_cache.shape[0]),
                                      int(heads) if rope is not None else 0, int(h), int(w), float(base),
                                      _stream(stream))
    _check("tsa_qkv_rows_to_cache", st)


def reuse_workspace_bytes(n_rows, heads):
    return int(lib().tsa_reuse_workspace_bytes(int(n_rows), int(heads)))


def timeripple_reuse(v, heads, head_dim, height, width, thetas, eff_out, workspace, *, src_out=None,
                     delta_out=None, stream=None):
    """Partial-score reuse on Q or K rows (tsa_timeripple_reuse); thetas = (time, height, width)."""
    dim = int(heads) * int(head_dim)
    n = v.shape[0]
    _need(v, "v", ("bf16",), cols=dim)
    _need(eff_out, "eff_out", ("bf16",), rows=n, cols=dim)
    _need(src_out, "src_out", ("i32",), numel=n * int(heads) * 3)
    _need(delta_out, "delta_out", ("f32",), numel=n * int(heads) * 3)
    th = (ctypes.c_float * 3)(*[float(t) for t in thetas])
    st = lib().tsa_timeripple_reuse(_ptr(v), int(v.shape[0]), int(heads), int(head_dim), int(height),
                                    int(width), ctypes.cast(th, ctypes.c_void_p), _ptr(eff_out), _ptr(src_out),
                                    _ptr(delta_out), _ptr(workspace),
                                    0 if workspace is None else workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _check("tsa_timeripple_reuse", st)


def timeripple_reuse_noalloc(v, heads, head_dim, height, width, thetas, eff_out, *, src_out=None,
                             delta_out=None, stream=None):
    """tsa_timeripple_reuse with the library's static scratch instead of a workspace
    (tsa_timeripple_reuse_noalloc): for callers that cannot allocate device memory."""
    dim = int(heads) * int(head_dim)
    n = v.shape[0]
    _need(v, "v", ("bf16",), cols=dim)
    _need(eff_out, "eff_out", ("bf16",), rows=n, cols=dim)
    _need(src_out, "src_out", ("i32",), numel=n * int(heads) * 3)
    _need(delta_out, "delta_out", ("f32",), numel=n * int(heads) * 3)
    th = (ctypes.c_float * 3)(*[float(t) for t in thetas])
    st = lib().tsa_timeripple_reuse_noalloc(_ptr(v), int(v.shape[0]), int(heads), int(head_dim), int(height),
                                            int(width), ctypes.cast(th, ctypes.c_void_p), _ptr(eff_out),
                                            _ptr(src_out), _ptr(delta_out), _stream(stream))
    _check("tsa_timeripple_reuse_noalloc", st)


def reuse_noalloc_max_token_heads() -> int:
    """Largest n_rows * heads timeripple_reuse_noalloc accepts."""
    return int(lib().tsa_reuse_noalloc_max_token_heads())


def token_scores(x_cur, x_ref, scores_out, *, ref_row_offset=0, score_kind=SCORE_REL_L1, stream=None):
    """a1 alone (tsa_token_scores)."""
    n, dim = x_cur.shape[0], x_cur.shape[1]
    _need(x_cur, "x_cur", ("bf16", "f32"), cols=dim)
    if x_ref is not None and x_ref.dtype != x_cur.dtype:
        raise ValueError("x_ref must have the dtype of x_cur")
    _need(x_ref, "x_ref", ("bf16", "f32"), rows=n, cols=dim)
    _need(scores_out, "scores_out", ("f32",), numel=n)
    st = lib().tsa_token_scores(_ptr(x_cur), _ptr(x_ref), int(ref_row_offset), int(x_cur.shape[0]),
                                int(x_cur.shape[1]), _dtype_code(x_cur), int(score_kind), _ptr(scores_out),
                                _stream(stream))
    _check("tsa_token_scores", st)


def qkv_active_rope(x, rows, n, w_qkv, heads, height, width, *, rope_base=10000.0, q_out=None, k_out, v_out,
                    out_is_cache=False, n_cache=0, eps=None, src_row_offset=0, sigma=0.0, stream=None):
    """qkv_active with 3D rotary positions on Q and K (tsa_qkv_active_rope)."""
    dim = x.shape[1]
    _need(x, "x", ("bf16", "f32"), cols=dim)
    _rows_index(rows, n, x.shape[0])
    _need(w_qkv, "w_qkv", ("bf16",), rows=3 * dim, cols=dim)
    _need(q_out, "q_out", ("bf16",), rows=n, cols=dim)
    if out_is_cache and k_out is not None and n_cache > k_out.shape[0]:
        raise ValueError(f"n_cache = {n_cache} exceeds the {k_out.shape[0]} rows of k_out")
    _need(k_out, "k_out", ("bf16",), rows=n_cache if out_is_cache else n, cols=dim)
    _need(v_out, "v_out", ("bf16",), rows=n_cache if out_is_cache else n, cols=dim)
    _need(eps, "eps", ("bf16",), rows=x.shape[0], cols=dim)
    st = lib().tsa_qkv_active_rope(
        _ptr(x), _dtype_code(x), int(x.shape[0]), _ptr(rows), int(n), int(x.shape[1]), _ptr(w_qkv),
        _ptr(q_out), _ptr(k_out), _ptr(v_out), 1 if out_is_cache else 0, int(n_cache), _ptr(eps),
        int(src_row_offset), float(sigma), int(heads), int(height), int(width), float(rope_base),
        _stream(stream))
    _check("tsa_qkv_active_rope", st)


def frame_causal_attention(q, k_cache, v_cache, n_q, heads, head_dim, q_tokens, frame_tokens, out, *,
                           out_rows=None, scale=0.0, lse_out=None, stream=None):
    """Frame-causal attention of the active queries (tsa_frame_causal_attention)."""
    dim = int(heads) * int(head_dim)
    _need(k_cache, "k_cache", ("bf16",), cols=dim)
    _need(v_cache, "v_cache", ("bf16",), rows=k_cache.shape[0], cols=dim)
    _need(q, "q", ("bf16",), rows=n_q, cols=dim)
    _need(out, "out", ("bf16",), rows=0 if out_rows is not None else n_q, cols=dim)
    _need(out_rows, "out_rows", ("i32",), numel=n_q)
    _need(lse_out, "lse_out", ("f32",), numel=int(heads) * int(n_q))
    _need(q_tokens, "q_tokens", ("i32",), numel=n_q)
    st = lib().tsa_frame_causal_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), int(n_q), int(k_cache.shape[0]), int(heads), int(head_dim),
        float(scale), _ptr(q_tokens), int(frame_tokens), _ptr(out), _ptr(out_rows), int(out.shape[0]),
        _ptr(lse_out), _stream(stream))
    _check("tsa_frame_causal_attention", st)
