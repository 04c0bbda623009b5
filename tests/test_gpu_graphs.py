"""The library's calls captured in HIP graphs (torch.cuda.CUDAGraph): every
launch goes to the caller's stream and nothing is allocated or cleared inside
a call, so a captured decode step, multi-token decode or prefill chunk
replays with whatever the static input buffers hold.  Each replay is checked
bitwise against the same call run eagerly, with eager work and
synchronisations between the replays."""
import pytest
import torch

from long_context_layers_amd import binding, inputs
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def test_decode_steps_replayed_from_a_graph():
    B, H, d, steps = 4, 8, 128, 6
    log(f"graph: decode step B{B} H{H} d{d}, {steps} replays")
    x = inputs.make_decode(B, H, d, steps, torch.bfloat16, seed=140, device=DEV)
    q, k, v = (torch.empty_like(x.q[0]) for _ in range(3))        # static inputs
    state = x.state.clone()
    out = torch.empty_like(x.q[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                                      # warm-up outside the capture
        binding.decode_step(q, k, v, x.slopes, state.clone(), out=torch.empty_like(out))
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.decode_step(q, k, v, x.slopes, state, out=out)
    state.copy_(x.state)                                            # capture ran nothing
    ref_state = x.state.clone()
    for t in range(steps):
        q.copy_(x.q[t]); k.copy_(x.k[t]); v.copy_(x.v[t])
        g.replay()
        ref = binding.decode_step(x.q[t], x.k[t], x.v[t], x.slopes, ref_state)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), t
        assert torch.equal(state, ref_state), t


def test_multi_token_decode_replayed_from_a_graph():
    B, H, T, d = 3, 4, 4, 64
    log(f"graph: multi-token decode B{B} H{H} T{T} d{d}")
    x = inputs.make_decode(B, H, d, 3 * T, torch.bfloat16, seed=141, device=DEV)
    toks = [(t.permute(1, 2, 0, 3).contiguous()) for t in (x.q, x.k, x.v)]   # [B,H,3T,d]
    q, k, v = (torch.empty((B, H, T, d), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    ncommit = torch.empty(B, dtype=torch.int32, device=DEV)
    state = x.state.clone()
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.decode_multi(q, k, v, x.slopes, state.clone(), n_commit=ncommit.zero_(),
                             out=torch.empty_like(out))
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.decode_multi(q, k, v, x.slopes, state, n_commit=ncommit, out=out)
    state.copy_(x.state)
    ref_state = x.state.clone()
    for r, counts in enumerate(([4, 1, 2], [0, 3, 4], [2, 2, 1])):
        for dst, src in zip((q, k, v), toks):
            dst.copy_(src[:, :, r * T:(r + 1) * T])
        ncommit.copy_(torch.tensor(counts, dtype=torch.int32))
        g.replay()
        ref = binding.decode_multi(q.clone(), k.clone(), v.clone(), x.slopes, ref_state,
                                   n_commit=ncommit.clone())
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        assert torch.equal(state, ref_state), r


def test_prefill_chunks_replayed_from_a_graph():
    # chunked prefill: one captured 192-token chunk replayed over a longer
    # sequence, the state carried from chunk to chunk inside the static buffer
    B, H, C, d, nchunk = 1, 4, 192, 128, 4
    log(f"graph: prefill chunks of {C} tokens B{B} H{H} d{d}, {nchunk} replays")
    x = inputs.make_prefill(B, H, C * nchunk, d, torch.bfloat16, seed=142, init_state=True,
                            device=DEV)
    q, k, v = (torch.empty((B, H, C, d), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    state = x.state.clone()
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.prefill(q, k, v, x.slopes, state.clone(), out=torch.empty_like(out))
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.prefill(q, k, v, x.slopes, state, out=out)
    state.copy_(x.state)
    ref_state = x.state.clone()
    for c in range(nchunk):
        sl = slice(c * C, (c + 1) * C)
        q.copy_(x.q[:, :, sl]); k.copy_(x.k[:, :, sl]); v.copy_(x.v[:, :, sl])
        g.replay()
        ref = binding.prefill(x.q[:, :, sl].contiguous(), x.k[:, :, sl].contiguous(),
                              x.v[:, :, sl].contiguous(), x.slopes, ref_state)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), c
        assert torch.equal(state, ref_state), c


def test_split_prefill_noalloc_replayed_from_a_graph():
    # the allocation-free split prefill (la_prefill_noalloc: its scratch is the
    # library's own, no allocation under capture) captured once and replayed,
    # each replay bitwise against the eager call on the same inputs
    B, H, N, d = 1, 32, 40000, 128
    if binding.prefill_workspace_bytes(B, H, N, d, DEV) == 0:
        pytest.skip("no sequence split planned on this device")
    log(f"graph: la_prefill_noalloc B{B} H{H} N{N} d{d}, 3 replays")
    lib = binding.load_library()
    x = inputs.make_prefill(B, H, N, d, torch.bfloat16, seed=143, init_state=True, device=DEV)
    out = torch.empty_like(x.q)
    state = x.state.clone()

    def call(o, st):
        rc = lib.la_prefill_noalloc(x.q.data_ptr(), x.k.data_ptr(), x.v.data_ptr(), x.slopes.data_ptr(),
                                    o.data_ptr(), st.data_ptr(), B, H, N, d,
                                    torch.cuda.current_stream().cuda_stream)
        assert rc == 0
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(torch.empty_like(out), state.clone())          # the first call finds the scratch
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, state)
    for r in range(3):
        state.copy_(x.state)
        g.replay()
        ref_state = x.state.clone()
        ref = torch.empty_like(out)
        call(ref, ref_state)                                 # eager, between the replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        assert torch.equal(state, ref_state), r


def test_fp32_split_prefill_replayed_from_a_graph():
    # la_prefill_f32_ws (prep, the fp32 segments, fold, fp32 correction) with a
    # workspace allocated before the capture
    B, H, N, d = 1, 16, 20000, 128
    ws = binding.prefill_f32_workspace_bytes(B, H, N, d, DEV)
    if ws == 0:
        pytest.skip("no fp32 sequence split planned on this device")
    log(f"graph: la_prefill_f32_ws B{B} H{H} N{N} d{d} (workspace {ws} B), 3 replays")
    lib = binding.load_library()
    x = inputs.make_prefill(B, H, N, d, torch.float32, seed=144, init_state=True, device=DEV)
    work = torch.empty(ws, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(x.q)
    state = x.state.clone()

    def call(o, st):
        rc = lib.la_prefill_f32_ws(x.q.data_ptr(), x.k.data_ptr(), x.v.data_ptr(), x.slopes.data_ptr(),
                                   o.data_ptr(), st.data_ptr(), B, H, N, d, work.data_ptr(), ws,
                                   torch.cuda.current_stream().cuda_stream)
        assert rc == 0
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(torch.empty_like(out), state.clone())
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, state)
    for r in range(3):
        state.copy_(x.state)
        g.replay()
        torch.cuda.synchronize()
        got, got_state = out.clone(), state.clone()
        ref_state = x.state.clone()
        ref = torch.empty_like(out)
        call(ref, ref_state)                                 # eager, between the replays
        torch.cuda.synchronize()
        assert torch.equal(got, ref), r
        assert torch.equal(got_state, ref_state), r


def test_outputs_only_packed_prefill_replayed_from_a_graph():
    # la_prefill_varlen_from_zero with null states: only the kernel, no state
    H, lens = 64, [64] * 300 + [1, 0, 200]
    log(f"graph: la_prefill_varlen_from_zero H{H}, {len(lens)} sequences, null states, 3 replays")
    x = inputs.make_varlen(H, lens, 128, torch.bfloat16, seed=145, init_state=False, device=DEV)
    out = torch.empty_like(x.q)

    def call(o):
        binding.prefill_varlen(x.q, x.k, x.v, x.slopes, x.cu_seqlens, None, out=o, from_zero=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(torch.empty_like(out))
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    for r in range(3):
        out.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = torch.empty_like(out)
        call(ref)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), r
