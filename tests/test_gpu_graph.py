"""A captured HIP graph of the simulated step gives, on every replay, the same
bits as the eager step (every kernel is deterministic and none of the library's
calls allocates, synchronises or clears memory with hipMemsetAsync)."""
import pytest
import torch

from gpu_util import bits_equal, say
from ulysses_inputs import seq_shards, small_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("sink,docs", [(False, None), (True, [[100, 1, 155]])])
def test_graph_replays_match_eager(sink, docs):
    from ulysses_sequence_attention_rank_amd import sim
    P, B, S, Hq, Hkv, D = 2, 1, 256, 8, 2, 128
    inp = small_case(41, P=P, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, sink=sink, doc_lengths=docs)
    dev = torch.device("cuda", 0)
    b = sim.allocate(seq_shards(inp.q, P).to(dev), seq_shards(inp.k, P).to(dev),
                     seq_shards(inp.v, P).to(dev), seq_shards(inp.dout, P).to(dev),
                     seq_shards(inp.positions, P).to(dev),
                     None if inp.sink is None else inp.sink.to(dev))
    outs = lambda: [t.clone() for t in (b.o_seq, b.lse, b.dq_seq, b.dk_seq, b.dv_seq, b.cu)
                    + ((b.dsink,) if sink else ())]
    say(f"graph test sink={sink}: eager step")
    sim.step(b, causal=True, window_left=63)
    torch.cuda.synchronize()
    eager = outs()
    say("capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sim.step(b, causal=True, window_left=63)
    for rep in range(3):
        # the program's own eager work between replays: scribble over the outputs
        for t in (b.o_seq, b.dq_seq, b.dk_seq, b.dv_seq, b.lse):
            t.fill_(7)
        torch.cuda.synchronize()
        say(f"replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for e, r in zip(eager, outs()):
            assert bits_equal(e, r), f"replay {rep} differs from the eager step"
