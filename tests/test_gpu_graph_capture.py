"""GPU test: kvq_decode_attention_static, the entry point for callers that
cannot allocate (code under stream capture among them), recorded into a HIP
graph through torch.cuda.CUDAGraph.  Nothing the call enqueues needs zeroed
memory, so the graph holds kernel launches only.  The graph is replayed
several times with the program's own eager work and synchronizations between
the replays (the output overwritten in between), and every replay must equal
the eager call bit for bit: the vector-ALU kernel alone and with its merge
launch, the matrix-core kernel with its in-launch merge, and the InnerQ
kernel."""
import math

import pytest
import torch

import decode_attention_token_amd as kvq
from workloads import Workload, gen_new_tokens, gen_prefill, gen_queries

pytestmark = pytest.mark.gpu


def _w(cid, B, Hq, Hkv, L, bits=2, G=32, R=128, sinks=0):
    return Workload(f"graph{cid}", cid, B, Hq, Hkv, 128, L, bits, G, R, 4, 10.0, 1, 1, 0, 0, sinks)


def _cache(w, scheme=kvq.KVQ_SCHEME_KIVI):
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda", steps=1)
    q = gen_queries(w, 0, "cuda", steps=1)[0].contiguous()
    if scheme == kvq.KVQ_SCHEME_INNERQ:
        cfg = kvq.make_innerq_config(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_q_heads,
                                     w.num_kv_heads, 128, w.context + 8)
    else:
        cap = ((w.context + 1 + w.residual - 1) // w.residual + 1) * w.residual
        cfg = kvq.make_config(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads, 128, cap)
    cache = kvq.KVCache(cfg, "cuda")
    cache.prefill(k, v)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    torch.cuda.synchronize()
    return cache, q


CASES = [
    ("mha-one-split", _w(701, 2, 8, 8, 1500), kvq.KVQ_SCHEME_KIVI, 1),
    ("mha-merge-launch", _w(702, 2, 8, 8, 3000), kvq.KVQ_SCHEME_KIVI, 5),
    ("gqa-matrix-cores", _w(703, 2, 16, 4, 3000), kvq.KVQ_SCHEME_KIVI, 0),
    ("innerq", _w(704, 1, 4, 4, 2500, 4, 64, 32, 4), kvq.KVQ_SCHEME_INNERQ, 3),
]


@pytest.mark.parametrize("name,w,scheme,splits", CASES, ids=[c[0] for c in CASES])
def test_static_attention_in_a_graph(name, w, scheme, splits):
    print(f"graph capture: {name}", flush=True)
    cache, q = _cache(w, scheme)
    scale = 1.0 / math.sqrt(128)
    want = cache.attention_static(q, scale, splits=splits)   # eager; also the first call on the device
    torch.cuda.synchronize()
    out = torch.empty_like(want)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cache.attention_static(q, scale, out=out, splits=splits)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        cache.attention_static(q, scale, out=out, splits=splits)
    filler = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        out.fill_(float("nan"))
        filler.mul_(1.0001)   # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r} differs from the eager call"
    # an eager call between replays leaves the graph's result unchanged
    again = cache.attention_static(q, scale, splits=splits)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(again, want) and torch.equal(out, want)
    del graph
