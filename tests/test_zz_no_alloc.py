"""The route entry point that allocates nothing (moe_route_topk_noalloc), against moe_route_topk.

Both are called through the C ABI with the same preallocated outputs; every output must be bit
for bit the same.  Two calls in a row on the same GPU, the second with fewer tokens, show that
the shared scratch left by the first call does not leak into the second.
"""

import numpy as np
import pytest
import torch

from gpu_util import note

pytestmark = pytest.mark.gpu


def _outputs(T, E, k, dev):
    z = lambda *shape, dt=torch.int32: torch.full(shape, -7, dtype=dt, device=dev)
    return dict(topk_idx=z(T, k), topk_gate=z(T, k, dt=torch.float32), probs=z(T, E, dt=torch.float32),
                counts=z(E), offsets=z(E + 1), offsets_pad=z(E + 1), dest=z(T, k), row_token=z(T * k))


def _args(logits, T, E, k, o):
    p = lambda t: t.data_ptr()
    return [p(logits), T, E, k, p(o["topk_idx"]), p(o["topk_gate"]), p(o["probs"]), p(o["counts"]),
            p(o["offsets"]), p(o["offsets_pad"]), 32, p(o["dest"]), p(o["row_token"])]


def _run_both(T, E, k, seed):
    from expert_ffn_layer_top_amd._lib import call, lib
    dev = torch.device("cuda:0")
    g = np.random.default_rng([seed, T, E, k])
    logits = torch.from_numpy(g.standard_normal((T, E), dtype=np.float32)).to(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ref = _outputs(T, E, k, dev)
    nbytes = lib.moe_route_workspace_bytes(T, E, k)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    call("moe_route_topk", *_args(logits, T, E, k, ref), ws.data_ptr(), nbytes, stream)
    out = _outputs(T, E, k, dev)
    torch.cuda.synchronize()
    call("moe_route_topk_noalloc", *_args(logits, T, E, k, out), stream)
    torch.cuda.synchronize()
    for key in ref:
        a, b = ref[key].cpu().numpy(), out[key].cpu().numpy()
        assert a.dtype == b.dtype and np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{key} differs (T={T})"
    # the outputs are the route's, not left-over fill values
    assert int(ref["offsets"][-1]) == T * k


@pytest.mark.parametrize("E,k", [(64, 4), (8, 2), (256, 16)])
def test_noalloc_route_matches_workspace_route_twice(E, k):
    # first call large (several blocks, a ragged last block), then a smaller one on the same GPU
    for T, seed in ((32768 + 37, 0), (300, 1)):
        note(f"route_topk_noalloc vs route_topk T={T} E={E} k={k}")
        _run_both(T, E, k, seed)
