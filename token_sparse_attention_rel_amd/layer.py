"""Driver of one pruned attention layer on one GPU: owns the persistent buffers
and sequences the C-ABI calls.  Token data is never touched on the host; the
only arithmetic here is scalar bookkeeping: the HSA schedule's active count per
step (the sum of the group sizes whose period divides the step, which sizes the
calls) and the Euler step sigma_{i+1} - sigma_i handed to the update kernel.

A step (HSA page §2.2) is: score + select + compact (select_active), QKV of
the active tokens with their K/V written straight into the cache rows
(qkv_active with the cache sync fused), attention of the active queries over
the whole cache with the outputs written straight to their token rows
(sparse_query_attention with the scatter fused).  ``fused=False`` runs the
same step with the standalone cache-sync and scatter kernels instead.
"""

from __future__ import annotations

import torch

from . import _binding as B


class PrunedAttentionLayer:
    def __init__(self, n: int, dim: int, heads: int, w_qkv: torch.Tensor, device="cuda", *,
                 split_attention: bool = True, rope=None, causal_frame_tokens=None, debug: bool = False):
        """``rope = (height, width, base)`` rotates Q and K by their tokens' 3D positions
        (the cache then holds rotated K); ``causal_frame_tokens`` makes the attention
        frame-causal (a query sees the frames up to its own).  ``debug``: every
        forward_active first reads the selection's active count back (one synchronisation)
        and raises if the count it was given differs."""
        if dim % heads:
            raise ValueError("dim must be a multiple of heads")
        self.rope = rope
        self.causal_frame_tokens = causal_frame_tokens
        self.debug = debug
        self.n, self.dim, self.heads = n, dim, heads
        self.head_dim = dim // heads
        self.device = torch.device(device)
        dev = self.device
        self.w_qkv = w_qkv.to(dev, torch.bfloat16).contiguous()
        bf = torch.bfloat16
        # persistent state: the per-layer KV cache and the output in token order
        self.k_cache = torch.zeros(n, dim, dtype=bf, device=dev)
        self.v_cache = torch.zeros(n, dim, dtype=bf, device=dev)
        self.out = torch.zeros(n, dim, dtype=bf, device=dev)
        # per-step scratch
        self.scores = torch.empty(n, dtype=torch.float32, device=dev)
        self.mask = torch.empty(n, dtype=torch.uint8, device=dev)
        self.idx = torch.empty(n, dtype=torch.int32, device=dev)
        self.pidx = torch.empty(n, dtype=torch.int32, device=dev)
        self.n_active = torch.empty(1, dtype=torch.int32, device=dev)
        self.q_a = torch.empty(n, dim, dtype=bf, device=dev)
        self._k_a = None
        self._v_a = None
        self._lif_mask = None
        self._o_a = None
        ws = B.select_workspace_bytes(n)
        self.workspace = torch.empty(max(ws, 16) + n, dtype=torch.uint8, device=dev)
        # partials of the attention's split last round, grown on demand
        self.split_attention = split_attention
        self._attn_ws = torch.empty(0, dtype=torch.uint8, device=dev)
        self._attn_ws_streams = []  # streams other than the allocating one that used it

    def attention_workspace(self, n_q: int, stream=None):
        """Workspace for attention of n_q active queries over the cache (None: no split),
        to be used on ``stream`` (None: the current stream)."""
        if not self.split_attention:
            return None
        with torch.cuda.device(self.device):
            need = B.attention_workspace_bytes(n_q, self.n, self.heads, self.head_dim)
        if need == 0:
            return None
        if self._attn_ws.numel() < need:
            # the old buffer may still be read by work queued on another stream: the
            # allocator must not hand it out again before that work is done
            for st in self._attn_ws_streams:
                self._attn_ws.record_stream(st)
            self._attn_ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            self._attn_ws_streams = []
        if stream is not None and stream not in self._attn_ws_streams:
            self._attn_ws_streams.append(stream)
        return self._attn_ws

    # ---------------------------------------------------------------- state

    def _qkv(self, x, rows, n, **kw):
        if self.rope is None:
            B.qkv_active(x, rows, n, self.w_qkv, **kw)
        else:
            h, w, base = self.rope
            B.qkv_active_rope(x, rows, n, self.w_qkv, self.heads, h, w, rope_base=base, **kw)

    def _attend(self, n_q, out, q_tokens, rows=None, stream=None):
        """Attention of the n_q queries in q_a (tokens q_tokens) over the cache."""
        if self.causal_frame_tokens is None:
            B.sparse_query_attention(self.q_a, self.k_cache, self.v_cache, n_q, self.heads, self.head_dim,
                                     out, out_rows=rows, workspace=self.attention_workspace(n_q, stream),
                                     stream=stream)
        else:
            B.frame_causal_attention(self.q_a, self.k_cache, self.v_cache, n_q, self.heads, self.head_dim,
                                     q_tokens, self.causal_frame_tokens, out, out_rows=rows, stream=stream)

    def _identity_rows(self):
        if getattr(self, "_iota", None) is None:
            self._iota = torch.arange(self.n, dtype=torch.int32, device=self.device)
        return self._iota

    def init_cache(self, x_prev: torch.Tensor, stream=None) -> None:
        """K/V cache = projections of every token of x_prev (the start of a run)."""
        self._qkv(x_prev, None, self.n, q_out=None, k_out=self.k_cache, v_out=self.v_cache, stream=stream)

    def _compact_bufs(self):
        if self._k_a is None:
            bf = torch.bfloat16
            self._k_a = torch.empty(self.n, self.dim, dtype=bf, device=self.device)
            self._v_a = torch.empty(self.n, self.dim, dtype=bf, device=self.device)
            self._o_a = torch.empty(self.n, self.dim, dtype=bf, device=self.device)
        return self._k_a, self._v_a, self._o_a

    # ---------------------------------------------------------------- steps

    def select(self, x_cur, x_ref=None, *, k=None, tau=None, mask=None, periods=None, step=0,
               ref_row_offset=0, score_kind=B.SCORE_REL_L1, stream=None) -> None:
        if mask is not None:
            B.select_active(None, None, 0, B.SELECT_MASK, aux_in=mask, mask_out=self.mask,
                            idx_out=self.idx, pidx_out=self.pidx, n_active_out=self.n_active,
                            n_rows=self.n, stream=stream)
        elif periods is not None:
            B.select_active(None, None, 0, B.SELECT_SCHEDULE, aux_in=periods, step=step,
                            mask_out=self.mask, idx_out=self.idx, pidx_out=self.pidx,
                            n_active_out=self.n_active, n_rows=self.n, stream=stream)
        else:
            mode = B.SELECT_TOPK if k is not None else B.SELECT_THRESHOLD
            B.select_active(x_cur, x_ref, ref_row_offset, mode, k=k or 0,
                            tau=0.0 if tau is None else tau, score_kind=score_kind,
                            scores_out=self.scores, mask_out=self.mask, idx_out=self.idx,
                            pidx_out=self.pidx, n_active_out=self.n_active, stream=stream)

    def forward_active(self, x_cur, n_active: int, *, fused=True, stream=None) -> None:
        """QKV of the selected tokens, cache sync, attention, scatter (after select)."""
        if self.debug:
            got = self._read_n_active(stream)
            if got != n_active:
                raise ValueError(f"forward_active: {n_active} active tokens given, the selection has {got}")
        if n_active == 0:
            return
        idx = self.idx
        if fused:
            self._qkv(x_cur, idx, n_active, q_out=self.q_a, k_out=self.k_cache, v_out=self.v_cache,
                      out_is_cache=True, n_cache=self.n, stream=stream)
            self._attend(n_active, self.out, idx, rows=idx, stream=stream)
        else:
            k_a, v_a, o_a = self._compact_bufs()
            self._qkv(x_cur, idx, n_active, q_out=self.q_a, k_out=k_a, v_out=v_a, stream=stream)
            B.kv_cache_sync(k_a, v_a, idx, n_active, self.k_cache, self.v_cache, stream=stream)
            self._attend(n_active, o_a, idx, stream=stream)
            B.scatter_out(o_a, idx, n_active, self.out, stream=stream)

    def _read_n_active(self, stream=None) -> int:
        """The active count of the last selection, read back after the selection queued on
        ``stream`` (None: the current stream) has finished: the copy runs on that stream."""
        if stream is None:
            return int(self.n_active.item())
        with torch.cuda.stream(stream):
            return int(self.n_active.item())

    def step_topk(self, x_cur, x_ref, k: int, *, fused=True, stream=None) -> None:
        """One step with a fixed active count k (no host synchronisation)."""
        self.select(x_cur, x_ref, k=k, stream=stream)
        self.forward_active(x_cur, k, fused=fused, stream=stream)

    def step_threshold(self, x_cur, x_ref, tau: float, *, fused=True, stream=None) -> int:
        """One step with s >= tau active; reads the active count back (one synchronisation)."""
        self.select(x_cur, x_ref, tau=tau, stream=stream)
        n_active = self._read_n_active(stream)
        self.forward_active(x_cur, n_active, fused=fused, stream=stream)
        return n_active

    def step_lipar(self, x, eps, hw: int, k: int, sigma: float, *, stream=None) -> None:
        """Inter-frame pass over a whole clip (LIPAR page §2.B-§2.C): score each token against
        the same location one frame earlier, keep the top k, project active tokens from their
        latent and pruned tokens from the recovered row, attend, scatter."""
        self.select(x, None, k=k, ref_row_offset=hw, stream=stream)
        self._lipar_forward(x, eps, hw, k, sigma, stream)

    def step_lipar_lif(self, x, eps, frames: int, hw: int, tau_short: float, tau_long: float,
                       sigma: float, *, score_kind=B.SCORE_ABS_L1, restore=True, stream=None) -> int:
        """Inter-frame pass with the long/short-term pruning mask (LIPAR page §2.B): a token is
        pruned when its change against the previous frame and against the last kept frame at
        its location are both below threshold.  Then the pass of step_lipar on that active
        set and, with ``restore``, the pruned rows of the output filled in from the previous
        frame (Dutch LIPAR page §2.D).  Reads the active count back (one synchronisation)."""
        if self._lif_mask is None:
            self._lif_mask = torch.empty(self.n, dtype=torch.uint8, device=self.device)
        B.lif_mask(x, frames, hw, tau_short, tau_long, self._lif_mask, score_kind=score_kind,
                   stream=stream)
        self.select(None, mask=self._lif_mask, stream=stream)
        k = self._read_n_active(stream)
        self._lipar_forward(x, eps, hw, k, sigma, stream)
        if restore:
            B.restore_frames(self.out, self._lif_mask, frames, hw, stream=stream)
        return k

    def _lipar_forward(self, x, eps, hw, k, sigma, stream):
        self._qkv(x, self.idx, k, q_out=self.q_a, k_out=self.k_cache, v_out=self.v_cache,
                  out_is_cache=True, n_cache=self.n, stream=stream)
        n_p = self.n - k
        if n_p:
            # recovered rows built once (gather), then projected into their cache rows: the
            # blend then runs once per row instead of once per output-feature tile
            rec = self._compact_bufs()[0]
            B.gather_rows(x, self.pidx, n_p, rec, eps=eps, src_row_offset=hw, sigma=sigma, stream=stream)
            B.qkv_rows_to_cache(rec, self.pidx, n_p, self.w_qkv, self.k_cache, self.v_cache, rope=self.rope,
                                heads=self.heads, stream=stream)
        if k:
            self._attend(k, self.out, self.idx, rows=self.idx, stream=stream)

    # ------------------------------------------------------- partial-score reuse

    def reuse_forward(self, x, thetas_q, thetas_k, *, stream=None) -> None:
        """Dense pass with Timeripple's partial-score reuse (Timeripple page, Metodología §2):
        rotated Q/K/V of every token, each channel group of each Q and K row taken from the
        neighbouring token whose group passes the similarity check (reuse_effective), then
        attention of the effective Q over the effective K in token order.  Needs ``rope``."""
        if self.rope is None:
            raise ValueError("partial-score reuse works on the rotary channel groups: construct with rope=")
        h, w, _ = self.rope
        bf = torch.bfloat16
        if getattr(self, "_q_eff", None) is None:
            self._q_eff = torch.empty(self.n, self.dim, dtype=bf, device=self.device)
            self._k_eff = torch.empty(self.n, self.dim, dtype=bf, device=self.device)
            self.src_q = torch.empty(self.n, self.heads, 3, dtype=torch.int32, device=self.device)
            self.src_k = torch.empty(self.n, self.heads, 3, dtype=torch.int32, device=self.device)
            self._reuse_ws = torch.empty(B.reuse_workspace_bytes(self.n, self.heads), dtype=torch.uint8,
                                         device=self.device)
        self._qkv(x, None, self.n, q_out=self.q_a, k_out=self.k_cache, v_out=self.v_cache, stream=stream)
        B.timeripple_reuse(self.q_a, self.heads, self.head_dim, h, w, thetas_q, self._q_eff, self._reuse_ws,
                           src_out=self.src_q, stream=stream)
        B.timeripple_reuse(self.k_cache, self.heads, self.head_dim, h, w, thetas_k, self._k_eff, self._reuse_ws,
                           src_out=self.src_k, stream=stream)
        B.sparse_query_attention(self._q_eff, self._k_eff, self.v_cache, self.n, self.heads, self.head_dim,
                                 self.out, workspace=self.attention_workspace(self.n, stream), stream=stream)

    # ------------------------------------------------------- sampling loop

    def dense_forward(self, x, stream=None) -> None:
        """Every token active: QKV of all rows straight into the cache, attention of all
        queries written in token order (no selection, no index indirection)."""
        self._qkv(x, None, self.n, q_out=self.q_a, k_out=self.k_cache, v_out=self.v_cache, stream=stream)
        self._attend(self.n, self.out, self._identity_rows(), stream=stream)

    def hsa_run(self, x, periods, sigmas, window: int, group_counts, group_periods, *,
                stream=None, on_step=None) -> None:
        """HSA page §2.1-§2.4: the sampling loop around the layer, on the state x (fp32 or
        bf16 [n, dim], updated in place).  Step i is dense inside the phase window (the first
        and last ``window`` steps), else it runs the tokens whose period divides i; the layer
        output, whose skipped rows keep their last value, is the cached velocity, and every
        token then advances by x <- x + (sigma_{i+1} - sigma_i) * v_hat.  ``periods`` is the
        device u8 period of every token (assign_groups); ``group_counts``/``group_periods``
        give the per-step active counts on the host, so no step synchronises."""
        steps = len(sigmas) - 1
        for i in range(steps):
            if i < window or i >= steps - window:
                self.dense_forward(x, stream=stream)
            else:
                self.select(None, periods=periods, step=i, stream=stream)
                self.forward_active(x, hsa_active_count(group_counts, group_periods, i),
                                    stream=stream)
            B.euler_update(x, self.out, float(sigmas[i + 1]) - float(sigmas[i]), stream=stream)
            if on_step is not None:
                on_step(i)


def hsa_active_count(group_counts, group_periods, step: int) -> int:
    """Active tokens at a global step of the HSA schedule (known on the host)."""
    return sum(c for c, p in zip(group_counts, group_periods) if p and step % p == 0)
