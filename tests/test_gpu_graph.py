"""The hot path captured in a HIP graph and replayed.

One verify call per temperature, one verify call with top-k / top-p and the
loss calls (E2E-TV with a probability target and with a logits target, and
the cross-entropy and KL comparators) are captured once into a graph on
torch's capture stream,
then replayed several times with eager work and synchronisations between the
replays; every replay must reproduce the eager outputs bit for bit. The
library enqueues kernels only (no memset nodes, no allocation, no host
sync), and the loss's call epoch advances inside the graph, so a replayed
call never takes an earlier replay's exchange words for its own."""

import numpy as np
import pytest
import torch

import lossless_verify_tv_amd as lv
from lossless_verify_tv_amd import synth

from .gpu_util import announce, device, logits_to_device, verify_inputs

pytestmark = pytest.mark.gpu


def _snapshot(tensors):
    return [t.detach().clone().cpu() for t in tensors]


def test_hot_path_replays_match_eager():
    dev = device()
    vcases = [synth.verify_case(3, temperature=T, batch=8, vocab=40000) for T in (0.0, 0.7, 1.0)]
    vins = [verify_inputs(c, dev) for c in vcases]
    B, K = vcases[0].k.shape[0], vcases[0].shape[1]
    vouts = [(torch.empty(B, dtype=torch.int32, device=dev),
              torch.empty(B, K + 1, dtype=torch.int32, device=dev),
              torch.empty(B, K, dtype=torch.float32, device=dev),
              torch.empty(B, dtype=torch.int32, device=dev)) for _ in vcases]
    lc = synth.loss_case(n_branches=6, width=7, vocab=30000)
    z = logits_to_device(lc.draft_logits, "bf16", dev)
    p = torch.from_numpy(lc.target_probs).to(dev)
    lg = synth.loss_logits_case(n_branches=6, width=7, vocab=30000)
    t = logits_to_device(lg.target_logits, "bf16", dev)
    N, W, V = lc.draft_logits.shape
    louts = [(torch.empty(1, dtype=torch.float32, device=dev),
              torch.empty(N, W, dtype=torch.float32, device=dev),
              torch.empty(N, W, V, dtype=torch.bfloat16, device=dev)) for _ in range(4)]
    vws = lv.new_workspace(lv.spec_verify_workspace_bytes(B, K, vcases[0].shape[2]), dev)
    lws = lv.new_workspace(max(lv.e2e_tv_loss_workspace_bytes(N, W, V),
                               lv.draft_loss_workspace_bytes(N, W, V),
                               lv.draft_loss_logits_workspace_bytes(N, W, V)), dev)
    tws = lv.new_workspace(lv.spec_verify_topkp_workspace_bytes(B, K, vcases[0].shape[2]), dev)
    top_k = torch.tensor([50, 3, 0, 200, 1, 40000, 7, 50][:B], dtype=torch.int32, device=dev)
    top_p = torch.tensor([0.9, 1.0, 0.8, 0.95, 1.0, 0.5, 0.99, 1.0][:B], dtype=torch.float32,
                         device=dev)
    touts = (torch.empty(B, dtype=torch.int32, device=dev),
             torch.empty(B, K + 1, dtype=torch.int32, device=dev),
             torch.empty(B, K, dtype=torch.float32, device=dev),
             torch.empty(B, dtype=torch.int32, device=dev))

    def run():
        for i, c in enumerate(vcases):
            lv.spec_verify(**vins[i], workspace=vws, out=vouts[i])
        lv.spec_verify_topkp(**vins[1], top_k=top_k, top_p=top_p, workspace=tws, out=touts)
        lv.e2e_tv_loss_fwd_bwd(z, p, workspace=lws, out=louts[0])
        lv.draft_loss_logits_fwd_bwd(z, t, 0.8, "e2e_tv", workspace=lws, out=louts[1])
        lv.draft_loss_fwd_bwd(z, p, "ce", workspace=lws, out=louts[2])
        lv.draft_loss_fwd_bwd(z, p, "kl", workspace=lws, out=louts[3])

    all_outs = [x for o in vouts for x in o] + list(touts) + [x for o in louts for x in o]
    # eager reference (on a side stream, as graph warm-up is done)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    ref = _snapshot(all_outs)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize(dev)
    for rep in range(4):
        for x in all_outs:           # poison the outputs: a replay must rewrite them
            x.fill_(7)
        scratch = torch.randn(1 << 20, device=dev).sum()   # eager work between replays
        torch.cuda.synchronize(dev)
        announce(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize(dev)
        got = _snapshot(all_outs)
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (rep, i)
        del scratch
    # an eager call after the replays still agrees (the workspace's epoch moved on)
    run()
    torch.cuda.synchronize(dev)
    got = _snapshot(all_outs)
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), ("eager", i)
