"""Opt-in canary bytes around the forward's workspace, o and final state
(api.chunk_fwd(..., guard=N)): no kernel writes outside its buffers, and the
guarded call returns the same bits as the plain one."""
import numpy as np
import pytest
import torch

from chunkwise_gated_delta_local_amd import api, synth
from gpu_common import to_dev

CASES = [
    ("cfg2", lambda: synth.generate(synth.WORKLOADS[2], seed=2), {}),
    ("cfg3", lambda: synth.generate(synth.WORKLOADS[3], seed=3), {}),
    ("varlen_ragged", lambda: synth.generate(synth.custom("g_var", B=1, T=0, Nk=2, Nv=4, dk=128, dv=64, dtype="bf16",
                                                          lengths=(1, 63, 64, 65, 200, 0, 130)), seed=5), {}),
    ("segmented", lambda: synth.generate(synth.custom("g_seg", B=1, T=0, Nk=1, Nv=2, dk=64, dv=128, dtype="bf16",
                                                      lengths=(700, 333)), seed=6), {"segment_chunks": 3}),
    ("f32_C32", lambda: synth.generate(synth.custom("g_f32", B=2, T=100, Nk=2, Nv=2, dk=32, dv=64, dtype="f32"),
                                       seed=7), {"chunk_size": 32}),
]


def run(inp, guard, extra):
    d = to_dev(inp)
    o, S = api.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"], initial_state=d["S0"],
                         cu_seqlens=d["cu_seqlens"], cu_seqlens_cpu=inp["cu_seqlens"], guard=guard, **extra)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.gpu
@pytest.mark.parametrize("name,make,extra", CASES, ids=[c[0] for c in CASES])
def test_forward_stays_inside_its_buffers(name, make, extra):
    inp = make()
    o0, S0 = run(inp, 0, extra)
    o1, S1 = run(inp, 4096, extra)          # raises if a canary byte changed
    assert torch.equal(o0, o1), name
    assert torch.equal(S0, S1), name
    print("%s: guarded call identical, canaries intact" % name, flush=True)


def test_guard_checker_reports_a_changed_byte():
    """The checker itself (CPU tensors): a byte changed just past a buffer is reported."""
    whole, inner = api._guarded(1000, 256, torch.device("cpu"))
    api._check_guards([("ws", whole)], 256)
    whole[256 + 1000 + 3] = 0
    with pytest.raises(RuntimeError, match="after the ws buffer"):
        api._check_guards([("ws", whole)], 256)
    whole[256 + 1000 + 3] = api._GUARD_BYTE
    whole[255] = 1
    with pytest.raises(RuntimeError, match="before the ws buffer"):
        api._check_guards([("ws", whole)], 256)
