"""The whole verify tree-step captured in HIP graphs: several replays, with
eager work and synchronisations between them, each equal to the eager step."""
import dataclasses

import numpy as np
import pytest
import torch

from speculative_decoding_05_amd import configs
from speculative_decoding_05_amd import step as st
from tests._lib import mb  # noqa: F401  (builds/loads the library)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16"])
def test_step_graph_replays_match_eager(name):
    if name == "small_bf16":
        cfg = dataclasses.replace(configs.CONFIGS["roofline_b16"], name="small_bf16", B=3, H=512, nh=4, dh=128,
                                  V=4000, L=300, K=4)
    else:
        cfg = configs.CONFIGS[name]
    tree = st.build_tree(cfg)
    host = st.host_inputs(cfg, tree.T)
    s = st.Step(cfg, tree, host, copies=2)
    s.heads()
    s.heads_vocab()
    s.topk_and_tokens()
    torch.cuda.synchronize()
    s.set_verify_logits(st.verify_logits_for(cfg, tree, s.topk_idx.cpu().numpy(), host["root_tok"]))
    outs = lambda: [t.clone() for t in (s.head_logits, s.topk_idx, s.tree_tok, s.attn, s.accept_len, s.best,
                                         s.next_tok, s.accepted)]
    eager = []
    for c in range(2):
        s.run(c)
        eager.append(outs())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s.run(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for c in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s.run(c)
        graphs.append(g)
    for rep in range(3):
        for c in range(2):
            graphs[c].replay()
            torch.cuda.synchronize()
            for a, b in zip(outs(), eager[c]):
                assert torch.equal(a, b), (rep, c)
            s.run(1 - c)                 # eager work between replays
            torch.cuda.synchronize()
    assert np.asarray(eager[0][4].cpu()).size == cfg.B
