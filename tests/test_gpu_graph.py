"""Graph capture of the block stack (HIP graph through torch.cuda.CUDAGraph):
the library enqueues no memset, copy or host wait on the block and attention
paths, so a forward + backward step can be captured, with the caller-owned
second stream of block_backward_overlap or on one stream.  Each replay, with
eager steps and synchronisations between the replays, must give the eager
step's output, input gradient and parameter gradients bit for bit."""
import pytest

from gpu_util import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("overlap", [True, False])
def test_block_stack_step_in_a_graph(overlap):
    require_gpu()
    import torch
    from decoder_only_transformer_block_amd import configs
    from decoder_only_transformer_block_amd.runtime import BlockStack, to_device
    cfg = configs.LLAMA_GQA.replace(B=2, T=384, L=2, C=512, NH=8, NKV=2, H=1408)
    announce(f"graph capture of a block-stack step, overlap={overlap}: {cfg.name} B={cfg.B} T={cfg.T} L={cfg.L}")
    ws = [configs.block_weights(cfg, l, perturb=True) for l in range(cfg.L)]
    x = to_device(configs.block_input(cfg), cfg.dtype)
    dy = to_device(configs.block_dout(cfg), cfg.dtype)
    st = BlockStack(cfg, ws, overlap=overlap)

    def step():
        st.forward(x)
        st.backward(dy)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the default stream, as capture requires
        step()
    torch.cuda.current_stream().wait_stream(side)
    st.zero_grads()
    step()
    torch.cuda.synchronize()
    ref_y = st.acts[cfg.L].clone()
    ref_dx = st.dx.clone()
    ref_g = [{k: v.clone() for k, v in g.items()} for g in st.grads]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        st.zero_grads()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.acts[cfg.L], ref_y), rep
        assert torch.equal(st.dx, ref_dx), rep
        for a, b in zip(st.grads, ref_g):
            for k in a:
                assert torch.equal(a[k], b[k]), (rep, k)
        st.zero_grads()
        step()                       # eager work between the replays
        torch.cuda.synchronize()
    del graph
    st.close()
