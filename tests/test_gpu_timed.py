"""The timed forward entry point (gdr_chunk_fwd_timed, used inside the
benchmark's timed region) computes what gdr_chunk_fwd computes, with every
stage event recorded or with only the two around the state pass (NULL
entries are skipped), and the recorded events bracket non-negative times."""
import pytest
import torch

from chunkwise_gated_delta_local_amd import api, synth
from gpu_common import to_dev

CASES = [
    ("bf16_fused", synth.custom("t_bf16", B=1, T=0, Nk=2, Nv=4, dk=128, dv=128, dtype="bf16",
                                lengths=(1, 63, 200, 130)), {}),
    ("bf16_segmented", synth.custom("t_seg", B=1, T=0, Nk=1, Nv=2, dk=64, dv=128, dtype="bf16",
                                    lengths=(700, 333)), {"segment_chunks": 3}),
    ("f32_C32", synth.custom("t_f32", B=2, T=100, Nk=2, Nv=2, dk=32, dv=64, dtype="f32"), {"chunk_size": 32}),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,w,extra", CASES, ids=[c[0] for c in CASES])
def test_timed_forward_matches_plain(name, w, extra):
    inp = synth.generate(w, seed=11)
    d = to_dev(inp)
    fwd = api.Forward(d["q"], d["k"], d["v"], d["beta"], g=d["g"], scale=inp["scale"], initial_state=d["S0"],
                      output_final_state=True, cu_seqlens=d["cu_seqlens"], cu_seqlens_cpu=inp["cu_seqlens"],
                      **extra)
    fwd()
    torch.cuda.synchronize()
    o_ref, s_ref = fwd.o.clone(), fwd.final_state.clone()
    full = [torch.cuda.Event(enable_timing=True) for _ in range(api.NUM_STAGES + 1)]
    pair = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in full + pair:
        e.record()
    torch.cuda.synchronize()
    for events in (full, [None] * 4 + pair + [None]):
        fwd.o.zero_()
        fwd.final_state.zero_()
        fwd.timed(events)
        torch.cuda.synchronize()
        assert torch.equal(fwd.o, o_ref), name
        assert torch.equal(fwd.final_state, s_ref), name
    times = [full[i].elapsed_time(full[i + 1]) for i in range(api.NUM_STAGES)]
    assert min(times) >= 0.0, times
    assert pair[0].elapsed_time(pair[1]) >= 0.0
    print("%s: timed calls identical; stage ms %s" % (name, ["%.4f" % t for t in times]), flush=True)
