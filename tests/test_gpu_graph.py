"""HIP graph capture of the entry points (the C ABI states they are safe to capture).

One graph captures fa_fwd, fa_bwd (caller workspace), fa_fwd_fp8, fa_paged_decode (caller
workspace), fa_paged_decode_noalloc (static scratch) and fa_paged_prefill (device-side plan,
attention and merge) twice: with fewer than 256 query rows per head (four-wave attention
workgroups) and with 256 (eight-wave ones).  Between replays the program's own eager work
rewrites the inputs in place -- new query values, new chunk lengths for the prefill (so its plan
changes from replay to replay), and on every other replay a key planted in the FP8 inputs that
sends that kernel's workgroup from its fixed-reference pass to the lagging one (a decision taken
on the device) -- and synchronises; every replay's outputs must equal, bitwise, those of eager
calls on the same inputs (the kernels are deterministic).  Nothing in the captured calls
allocates: outputs and workspaces are made beforehand.
"""

import pytest
import torch

from io_aware_attention_02_amd import (fa_bwd, fa_bwd_workspace_bytes, fa_fwd, fa_fwd_fp8,
                                       fa_paged_decode, fa_paged_decode_noalloc,
                                       fa_paged_decode_workspace_bytes, fa_paged_prefill,
                                       fa_paged_prefill_workspace_bytes)
from io_aware_attention_02_amd.inputs import (fp8_inputs, output_gradient, paged_decode_inputs,
                                              paged_prefill_inputs, prefill_inputs)

from gpu_common import device, say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_calls():
    dev = device()
    say("graph capture: fa_fwd, fa_bwd, fa_fwd_fp8, fa_paged_decode, fa_paged_decode_noalloc, "
        "fa_paged_prefill")
    # Forward: causal, grouped heads, one ragged sequence.
    q, k, v, _ = prefill_inputs(2, 8, 2, 300, 128, "bf16", seed=501)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    lens = torch.tensor([300, 177], dtype=torch.int32, device=dev)
    o, lse = torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    # Backward of the same attention (its O and LSE from an eager forward; dO rewritten per replay).
    bo, blse = fa_fwd(q, k, v, causal=True, seq_lens=lens)
    gout = output_gradient(2, 8, 300, 128, seed=506).to(dev)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(fa_bwd_workspace_bytes(2, 8, 300), dtype=torch.uint8, device=dev)
    # FP8 forward: 4 heads of 1031 keys; row 700 of head 0 can be given a dominating key 650.
    f8q, f8k, f8v, f8s, _ = fp8_inputs(1, 4, 2, 1031, 128, seed=507)
    f8q, f8k, f8v = f8q.to(dev), f8k.to(dev), f8v.to(dev)
    f8k_plain, f8k_planted = f8k.clone(), f8k.clone()
    f8k_planted[0, 0, 650] = f8q[0, 0, 700]
    f8o, f8l = torch.empty(f8q.shape, dtype=torch.bfloat16, device=dev), \
        torch.empty(f8q.shape[:3], dtype=torch.float32, device=dev)
    # Decode: 8 sequences of up to 3000 tokens.
    dq, kc, vc, table, sl = paged_decode_inputs(8, 32, 8, 128, 16, len_lo=1, len_hi=3000, seed=502)
    dq, kc, vc, table, sl = (t.to(dev) for t in (dq, kc, vc, table, sl))
    do, dl = torch.empty_like(dq), torch.empty(dq.shape[:2], dtype=torch.float32, device=dev)
    do2, dl2 = torch.empty_like(do), torch.empty_like(dl)
    dws = torch.empty(fa_paged_decode_workspace_bytes(8, 32, 128, table.shape[1], 16),
                      dtype=torch.uint8, device=dev)
    # Chunked prefill: contexts of a few thousand tokens, chunks that change per replay.
    S, Qmax = 4, 96
    pq, pkc, pvc, ptb, psl, pql = paged_prefill_inputs(S, 32, 8, 128, Qmax, seed=503,
                                                       seq_lens=[3000, 1500, 700, 96],
                                                       q_lens=[96, 40, 1, 96])
    pq, pkc, pvc, ptb, psl, pql = (t.to(dev) for t in (pq, pkc, pvc, ptb, psl, pql))
    po, pl = torch.empty_like(pq), torch.empty(pq.shape[:3], dtype=torch.float32, device=dev)
    pws = torch.empty(fa_paged_prefill_workspace_bytes(S, Qmax, 32, 8, 128, ptb.shape[1]),
                      dtype=torch.uint8, device=dev)
    # The same with 256 query rows per head (eight-wave work items).
    W = 256
    wq, wkc, wvc, wtb, wsl, wql = paged_prefill_inputs(2, 8, 2, 128, W, seed=505,
                                                       seq_lens=[4000, 600], q_lens=[256, 130])
    wq, wkc, wvc, wtb, wsl, wql = (t.to(dev) for t in (wq, wkc, wvc, wtb, wsl, wql))
    wo, wl = torch.empty_like(wq), torch.empty(wq.shape[:3], dtype=torch.float32, device=dev)
    wws = torch.empty(fa_paged_prefill_workspace_bytes(2, W, 8, 2, 128, wtb.shape[1]),
                      dtype=torch.uint8, device=dev)

    def captured():
        fa_fwd(q, k, v, o, lse, causal=True, seq_lens=lens)
        fa_bwd(q, k, v, bo, blse, gout, gq, gk, gv, causal=True, seq_lens=lens, workspace=bws)
        fa_fwd_fp8(f8q, f8k, f8v, *f8s, o=f8o, lse=f8l)
        fa_paged_decode(dq, kc, vc, table, sl, do, dl, workspace=dws)
        fa_paged_decode_noalloc(dq, kc, vc, table, sl, do2, dl2)
        fa_paged_prefill(pq, pkc, pvc, ptb, psl, pql, po, pl, workspace=pws)
        fa_paged_prefill(wq, wkc, wvc, wtb, wsl, wql, wo, wl, workspace=wws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        captured()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured()
    torch.cuda.synchronize()

    g = torch.Generator(device="cpu").manual_seed(504)
    chunk_sets = [[96, 40, 1, 96], [1, 96, 50, 0], [33, 2, 96, 17], [96, 96, 96, 96]]
    wide_sets = [[256, 130], [3, 256], [200, 0], [256, 256]]
    for rep, chunks in enumerate(chunk_sets):
        # Eager work between replays: new inputs, written in place.
        q.copy_(torch.randn(q.shape, generator=g).to(torch.bfloat16))
        dq.copy_(torch.randn(dq.shape, generator=g).to(torch.bfloat16))
        pq.copy_(torch.randn(pq.shape, generator=g).to(torch.bfloat16))
        pql.copy_(torch.tensor(chunks, dtype=torch.int32))
        wq.copy_(torch.randn(wq.shape, generator=g).to(torch.bfloat16))
        wql.copy_(torch.tensor(wide_sets[rep], dtype=torch.int32))
        gout.copy_(torch.randn(gout.shape, generator=g).to(torch.bfloat16))
        f8k.copy_(f8k_planted if rep % 2 else f8k_plain)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, do, dl, do2, dl2, po, pl, wo, wl, gq, gk, gv, f8o, f8l)]
        eo, el = fa_fwd(q, k, v, causal=True, seq_lens=lens)
        egq, egk, egv = fa_bwd(q, k, v, bo, blse, gout, causal=True, seq_lens=lens)
        e8o, e8l = fa_fwd_fp8(f8q, f8k, f8v, *f8s)
        edo, edl = fa_paged_decode(dq, kc, vc, table, sl)
        eo8, el8 = fa_paged_prefill(pq, pkc, pvc, ptb, psl, pql)
        ewo, ewl = fa_paged_prefill(wq, wkc, wvc, wtb, wsl, wql)
        torch.cuda.synchronize()
        names = ["fwd O", "fwd LSE", "decode O", "decode LSE", "noalloc O", "noalloc LSE",
                 "prefill O", "prefill LSE", "wide prefill O", "wide prefill LSE",
                 "bwd dQ", "bwd dK", "bwd dV", "fp8 O", "fp8 LSE"]
        want = [eo, el, edo, edl, edo, edl, eo8, el8, ewo, ewl, egq, egk, egv, e8o, e8l]
        for name, a, b in zip(names, got, want):
            assert torch.equal(a, b), f"replay {rep} (chunks {chunks}): {name} differs from eager"
        assert torch.isfinite(f8o).all()
        say(f"  replay {rep}, chunks {chunks} and {wide_sets[rep]}, FP8 key planted {bool(rep % 2)}: "
            "every output equals the eager call")
