"""HIP-graph capture of the library's calls.

Every entry point only enqueues kernels on the caller's stream (no device
allocation, no memset, no host synchronisation), so a caller can capture its
calls into a graph and replay them.  The graph below holds a bf16 forward with
key padding and grouped heads, its backward (caller-owned scratch), the fp8
preparation of q, k and v (rotated amax and quantisation, transposed V: the
amax is cleared by a kernel of its own, not a memset) and an fp8 forward on the
prepared bytes.  It is replayed several times, with eager work (every output
overwritten) and synchronisations between the replays, and every replay must
reproduce the eager results bit for bit.  (The fp8 forward takes its descales
as host values: the graph bakes in the ones of the eager run, which the replays
recompute identically.)
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_14_amd as attn
from workloads import make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load_library()
    return torch.device("cuda:0")


def ok(status, what):
    assert status == attn.ATTN_OK, f"{what}: {attn.attn_status_str(status)}"


@pytest.mark.parametrize("causal", [False, True])
def test_captured_calls_replay_like_eager(dev, causal):
    B, H, Hkv, N, d = 2, 4, 2, 300, 128
    q, k, v, kl = make_qkv(B, H, Hkv, N, d, "bf16", seed=77, padded=True)
    q, k, v, kl = q.to(dev), k.to(dev), v.to(dev), kl.to(dev)
    scale = float(np.float32(1 / math.sqrt(d)))
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(78)).to(torch.bfloat16).to(dev)
    signs = attn.hadamard_signs(d, seed=5, device=dev)
    n16 = (N + 15) // 16 * 16
    c = int(causal)
    klp = kl.data_ptr()

    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((2, B, H, N), dtype=torch.float32, device=dev)
    scal = torch.zeros(24, dtype=torch.float32, device=dev)  # amax / descale of q, k, v, 16 bytes apart
    q8 = torch.empty(q.shape, dtype=torch.float8_e4m3fn, device=dev)
    k8 = torch.empty(k.shape, dtype=torch.float8_e4m3fn, device=dev)
    vt8 = torch.empty((B, Hkv, d, n16), dtype=torch.float8_e4m3fn, device=dev)
    o8, lse8 = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=dev)
    outputs = [o, lse, dq, dk, dv, scal, q8, k8, vt8, o8, lse8]
    ptr = [scal[4 * i:].data_ptr() for i in range(6)]

    def prepare(stream):
        ok(attn.attn_fwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              B, H, Hkv, N, d, scale, c, klp, stream), "forward")
        ok(attn.attn_bwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                              lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                              B, H, Hkv, N, d, scale, c, klp, stream), "backward")
        for x, x8, i in ((q, q8, 0), (k, k8, 2)):
            rows = x.numel() // d
            ok(attn.attn_fp8_amax(x.data_ptr(), signs.data_ptr(), rows, d, ptr[i], stream), "amax")
            ok(attn.attn_fp8_quantize(x.data_ptr(), signs.data_ptr(), rows, d, ptr[i], x8.data_ptr(), ptr[i + 1],
                                      stream), "quantize")
        ok(attn.attn_fp8_amax(v.data_ptr(), None, B * Hkv * N, d, ptr[4], stream), "amax of v")
        ok(attn.attn_fp8_quantize_vt(v.data_ptr(), B * Hkv, N, d, ptr[4], vt8.data_ptr(), ptr[5], stream),
           "quantize_vt")

    def fp8_forward(stream, descales):
        ok(attn.attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), o8.data_ptr(), lse8.data_ptr(),
                             *descales, B, H, Hkv, N, d, scale, c, klp, stream), "fp8 forward")

    # eager run
    cur = torch.cuda.current_stream(dev)
    prepare(cur.cuda_stream)
    torch.cuda.synchronize()
    descales = tuple(float(scal[i].item()) for i in (4, 12, 20))
    fp8_forward(cur.cuda_stream, descales)
    torch.cuda.synchronize()
    eager = [t.view(torch.uint8).clone() for t in outputs]
    assert torch.isfinite(o.float()).all() and torch.isfinite(dq.float()).all()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s = torch.cuda.current_stream(dev).cuda_stream
        prepare(s)
        fp8_forward(s, descales)
    torch.cuda.synchronize()

    for rep in range(4):
        for t in outputs:  # eager work between replays: every output overwritten
            t.view(torch.uint8).fill_(0xFF if rep % 2 == 0 else 0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outputs, eager)):
            if t is scal:  # only the six amax / descale slots are outputs; the rest is padding
                t, e = t[0::4].contiguous(), e.view(torch.float32)[0::4].contiguous().view(torch.uint8)
            assert torch.equal(t.view(torch.uint8), e), f"replay {rep}: output {i} differs from the eager run"
