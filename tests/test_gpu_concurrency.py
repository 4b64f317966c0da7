"""Two pruned layers stepping at the same time on two streams, driven from two host threads: the
library keeps no per-call state (only a per-device cache of the attention kernel's resident
workgroup count, filled under first use), so every call on either stream gives what the same
call gives alone, bit for bit.  Streams at the default priority."""

from __future__ import annotations

import threading

import pytest
import torch

import gpu_util as G
from workloads import configs, generate
from workloads.configs import scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.need_gpu()


def _inputs(seed):
    cfg = scaled(configs.get_config("wan13b"), frames=4, height=20, width=26, dim=768, heads=6)
    inp = generate.step_inputs(cfg, seed)
    dev = torch.device("cuda")
    return cfg, inp["w_qkv"].to(dev), inp["x_prev"].to(dev), inp["x_cur"].to(dev)


def _layer(t, cfg, w, xp):
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, w, device=torch.device("cuda"))
    layer.init_cache(xp)
    return layer


def test_two_layers_on_two_streams_from_two_threads():
    import token_sparse_attention_rel_amd as t

    cases = [_inputs(1), _inputs(2)]
    ks = [cases[0][0].n_active, cases[1][0].n_active // 2]
    # each layer stepped alone
    want = []
    for (cfg, w, xp, xc), k in zip(cases, ks):
        layer = _layer(t, cfg, w, xp)
        for _ in range(3):
            layer.step_topk(xc, xp, k)
        torch.cuda.synchronize()
        want.append((layer.idx[:k].clone(), layer.k_cache.clone(), layer.out.clone()))
    print(f"  N={cases[0][0].n} D={cases[0][0].dim} k={ks}", flush=True)
    # both at once: one host thread and one stream each
    layers = [_layer(t, cfg, w, xp) for (cfg, w, xp, _) in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def run(i):
        try:
            cfg, w, xp, xc = cases[i]
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    layers[i].step_topk(xc, xp, ks[i], stream=streams[i])
        except Exception as e:  # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, k in enumerate(ks):
        assert torch.equal(layers[i].idx[:k], want[i][0]), i
        assert torch.equal(layers[i].k_cache, want[i][1]), i
        assert torch.equal(layers[i].out, want[i][2]), i
