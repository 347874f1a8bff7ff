"""attn_bwd_bf16_noalloc (the backward entry point whose scratch is built into
the library) against attn_bwd_bf16 (caller-owned scratch), through the C ABI.

Both run the same kernels on the same scratch contents (the first kernel
writes every value the second reads), so the gradients must be bitwise equal;
that is stricter than the oracle bar the backward pass is held to elsewhere.
Two calls in a row, the second on a smaller problem, so that a leftover of the
first call's scratch contents would show.  The no-alloc calls must allocate
nothing through torch's allocator (the library allocates nothing at all).
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_14_amd as attn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load_library()
    return torch.device("cuda:0")


def _case(dev, B, H, Hkv, N, d, causal, key_lens, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16).to(dev)
    do = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev)
    kl = None if key_lens is None else torch.tensor(key_lens, dtype=torch.int32, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = attn.forward(q, k, v, scale=scale, causal=causal, key_lens=kl)
    return q, k, v, do, kl, scale, o, lse


def test_noalloc_backward_matches_the_allocating_entry_point(dev):
    stream = torch.cuda.current_stream(dev).cuda_stream
    # the second problem is smaller (fewer rows of scratch) than the first
    cases = [(2, 8, 2, 1000, 128, True, [1000, 613], 1), (1, 4, 4, 300, 64, False, None, 2)]
    for B, H, Hkv, N, d, causal, key_lens, seed in cases:
        print(f"noalloc backward: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} key_lens={key_lens}", flush=True)
        q, k, v, do, kl, scale, o, lse = _case(dev, B, H, Hkv, N, d, causal, key_lens, seed)
        ref = attn.backward(q, k, v, o, lse, do, scale=scale, causal=causal, key_lens=kl)
        got = (torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan")))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        st = attn.attn_bwd_bf16_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                        lse.data_ptr(), got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(),
                                        B, H, Hkv, N, d, scale, int(causal),
                                        None if kl is None else kl.data_ptr(), stream)
        assert st == attn.ATTN_OK, attn.attn_status_str(st)
        torch.cuda.synchronize()
        assert torch.cuda.max_memory_allocated(dev) == before, "the no-alloc call allocated through torch"
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"{name} differs from attn_bwd_bf16's"
        # the binding's no-alloc form with caller-given outputs: the same again
        out = tuple(torch.empty_like(t) for t in got)
        attn.backward(q, k, v, o, lse, do, scale=scale, causal=causal, key_lens=kl, out=out, builtin_scratch=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), out, ref):
            assert torch.equal(a, b), f"{name} (binding) differs from attn_bwd_bf16's"


def test_noalloc_backward_rejects_problems_beyond_its_scratch(dev):
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device=dev)
    N = attn.ATTN_NOALLOC_SCRATCH_FLOATS // 2 + 1  # 2·B·H·N one float past the limit (pointers are not read)
    st = attn.attn_bwd_bf16_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                    q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                    1, 1, 1, N, 64, 0.125, 0, None, None)
    assert st == attn.ATTN_ERR_SCRATCH


def test_noalloc_backward_replays_in_a_graph(dev):
    """The callers this entry point is for include those that capture their
    calls into a graph.  After one eager call (which looks up the scratch
    array's address), the call is captured and replayed four times; between
    replays the outputs are overwritten and another problem runs through the
    same entry point (so the shared scratch holds other contents), and every
    replay must give the eager gradients bit for bit."""
    q, k, v, do, kl, scale, o, lse = _case(dev, 1, 4, 2, 500, 128, True, [437], 3)
    q2, k2, v2, do2, kl2, scale2, o2, lse2 = _case(dev, 2, 2, 1, 200, 64, False, [200, 150], 4)
    grads = tuple(torch.empty_like(t) for t in (q, k, v))
    other = tuple(torch.empty_like(t) for t in (q2, k2, v2))

    def call(stream):
        st = attn.attn_bwd_bf16_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                        lse.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                                        grads[2].data_ptr(), 1, 4, 2, 500, 128, scale, 1, kl.data_ptr(), stream)
        assert st == attn.ATTN_OK, attn.attn_status_str(st)

    call(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    eager = [g.clone() for g in grads]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    for rep in range(4):
        for g in grads:
            g.fill_(float("nan"))
        attn.backward(q2, k2, v2, o2, lse2, do2, scale=scale2, key_lens=kl2, out=other, builtin_scratch=True)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), grads, eager):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
