"""The pruned layer step at the headline shape (32760 tokens of 1536, 12 heads of 128) captured
once as a HIP graph and replayed: top-k selection, QKV with the cache sync fused, attention with
the scatter fused.  The library queues no memset and never synchronises, so the step captures;
every replay, with eager work of the program between replays, must give the eager step's index
list, caches and outputs bit for bit.  k = 9828 runs one workgroup per query tile; k = 8190 leaves
the last round of tiles partly idle, so the split schedule (workspace partials + merge) runs too."""

from __future__ import annotations

import pytest
import torch

import gpu_util as G
from workloads import configs, generate

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.need_gpu()


@pytest.mark.parametrize("k", [9828, 8190])
def test_layer_step_replays_as_a_graph(k):
    import token_sparse_attention_rel_amd as t

    cfg = configs.get_config("wan13b")
    inp = generate.step_inputs(cfg, 0)
    dev = torch.device("cuda")
    w = inp["w_qkv"].to(dev)
    xp = inp["x_prev"].to(dev)
    xc = inp["x_cur"].to(dev)
    print(f"  N={cfg.n} D={cfg.dim} heads={cfg.heads} k={k}", flush=True)

    eager = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, w, device=dev)
    eager.init_cache(xp)
    eager.step_topk(xc, xp, k)
    torch.cuda.synchronize()
    want = (eager.idx[:k].clone(), eager.k_cache.clone(), eager.v_cache.clone(), eager.out.clone())
    split = eager.attention_workspace(k) is not None
    print(f"  split schedule: {split}", flush=True)
    assert split == (k == 8190)

    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, w, device=dev)
    layer.init_cache(xp)
    layer.step_topk(xc, xp, k)  # warm-up: workspaces allocated, device queries cached
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.step_topk(xc, xp, k)
    for rep in range(3):
        # eager work between the replays: the caches start over, the outputs are cleared
        layer.init_cache(xp)
        layer.out.zero_()
        layer.idx.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.idx[:k], want[0]), rep
        assert torch.equal(layer.k_cache, want[1]) and torch.equal(layer.v_cache, want[2]), rep
        assert torch.equal(layer.out, want[3]), rep
