"""C-ABI library: loads, exports every declared symbol, validates on the host.

No device work: gdr_validate and gdr_chunk_fwd_workspace_size are host-only,
and gdr_chunk_fwd is only called with arguments it must reject before any
launch.
"""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from chunkwise_gated_delta_local_amd import api
    if not os.path.exists(api.library_path()):
        from chunkwise_gated_delta_local_amd.build import build
        build()
    return api.load_library()


def declared_functions():
    """Every function declared in include/*.h."""
    names = set()
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names.update(re.findall(r"\b(gdr_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 7, names
    for n in names:
        assert hasattr(lib, n), n
    from chunkwise_gated_delta_local_amd import api
    assert sorted(api.EXPORTED) == names


def prob(**kw):
    from chunkwise_gated_delta_local_amd import api
    base = dict(batch=2, seq_len=100, Nk=2, Nv=4, dk=64, dv=64, num_seqs=2, io_dtype=api.GDR_BF16)
    base.update(kw)
    return api.make_problem(**base)


def status(p, cu=None):
    from chunkwise_gated_delta_local_amd import api
    return api.validate(p, cu)


def test_validate_accepts_good_problems(lib):
    assert status(prob()) == 0
    assert status(prob(batch=1, seq_len=10, num_seqs=3), [0, 0, 4, 10]) == 0
    assert status(prob(batch=1, seq_len=0, num_seqs=1), [0, 0]) == 0
    for d in (32, 64, 128):
        assert status(prob(dk=d, dv=128 if d == 32 else 32)) == 0
    for C in (16, 32, 64):
        assert status(prob(chunk_size=C)) == 0


def test_workspace_scales_with_chunk_size(lib):
    """Five-kernel intermediates scale with C (A rows of C entries, W and U of
    C positions per chunk, more chunks for smaller C); bf16 with C = 64 takes
    the fused path's smaller workspace."""
    from chunkwise_gated_delta_local_amd import api
    f32 = {C: api.workspace_size(prob(seq_len=4096, io_dtype=api.GDR_F32, beta_dtype=api.GDR_F32, chunk_size=C))
           for C in (16, 32, 64)}
    assert f32[16] > f32[64] and f32[32] > f32[64]
    bf = {C: api.workspace_size(prob(seq_len=4096, chunk_size=C)) for C in (16, 32, 64)}
    assert bf[64] < bf[32] and bf[64] < bf[16]


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), 2), (dict(seq_len=-1), 2), (dict(Nk=3, Nv=4), 2), (dict(Nk=0), 2),
    (dict(io_dtype=7), 3), (dict(beta_dtype=1, io_dtype=0), 3),
    (dict(dk=48), 4), (dict(dv=256), 4), (dict(chunk_size=48), 4), (dict(chunk_size=128), 4),
    (dict(num_seqs=3), 2),
])
def test_validate_rejects(lib, kw, code):
    assert status(prob(**kw)) == code


@pytest.mark.parametrize("cu,code", [
    ([1, 5, 10], 5), ([0, 6, 5], 5), ([0, 4, 9], 5),
])
def test_validate_rejects_bad_seqlens(lib, cu, code):
    assert status(prob(batch=1, seq_len=10, num_seqs=2), cu) == code


def test_varlen_requires_batch_one(lib):
    assert status(prob(batch=2, seq_len=10, num_seqs=2), [0, 5, 10]) == 5


def test_error_message_and_status_strings(lib):
    assert status(prob(dk=48)) == 4
    assert b"head dims" in lib.gdr_last_error_message()
    for s in range(8):
        assert lib.gdr_status_string(s)


def test_workspace_size_grows_with_tokens(lib):
    from chunkwise_gated_delta_local_amd import api
    a = api.workspace_size(prob(seq_len=64))
    b = api.workspace_size(prob(seq_len=6400))
    assert 0 < a < b
    assert api.workspace_size(prob(seq_len=0)) > 0


def test_fwd_rejects_before_launch(lib):
    """Bad arguments come back as status codes with no device work."""
    from chunkwise_gated_delta_local_amd import api
    if torch.cuda.is_available():
        pytest.skip("passes placeholder addresses; host-logic test for machines without a GPU")
    p = prob()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: rejected first
    args = [ctypes.byref(p), fake, fake, fake, None, fake, ctypes.c_float(1.0), None, None, None, fake, None]
    # missing workspace
    assert lib.gdr_chunk_fwd(*args, None, ctypes.c_size_t(0), None) == 6
    # too-small workspace
    assert lib.gdr_chunk_fwd(*args, fake, ctypes.c_size_t(256), None) == 6
    # misaligned tensor
    bad = list(args)
    bad[1] = ctypes.c_void_p((1 << 20) + 4)
    assert lib.gdr_chunk_fwd(*bad, fake, ctypes.c_size_t(1 << 40), None) == 2
    # only one of the two cu_seqlens copies
    bad = list(args)
    bad[8] = fake
    assert lib.gdr_chunk_fwd(*bad, fake, ctypes.c_size_t(1 << 40), None) == 1
    # required pointer missing
    bad = list(args)
    bad[2] = null
    assert lib.gdr_chunk_fwd(*bad, fake, ctypes.c_size_t(1 << 40), None) == 1


def test_debug_rejects_misaligned_pair_buffers_before_launch(lib):
    """gdr_chunk_fwd_debug expands the packed T and score-block pairs with
    16-byte accesses: a misaligned T or P buffer is refused before any work."""
    from chunkwise_gated_delta_local_amd import api
    if torch.cuda.is_available():
        pytest.skip("passes placeholder addresses; host-logic test for machines without a GPU")
    p = prob()
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: rejected first
    args = [ctypes.byref(p), fake, fake, fake, None, fake, ctypes.c_float(1.0), None, None, None, fake, None,
            fake, ctypes.c_size_t(1 << 40), None]
    for field in ("T", "P"):
        dbg = api.Intermediates()
        setattr(dbg, field, (1 << 20) + 8)
        assert lib.gdr_chunk_fwd_debug(*args, ctypes.byref(dbg)) == 2, field
        assert b"16-byte aligned" in lib.gdr_last_error_message()
    assert lib.gdr_chunk_fwd_debug(*args, None) == 1


def test_binding_refuses_cpu_tensors(lib):
    from chunkwise_gated_delta_local_amd import api
    q = torch.zeros(1, 8, 1, 32)
    with pytest.raises(ValueError):
        api.chunk_fwd(q, q, q, torch.zeros(1, 8, 1))


def test_validate_out_dtype(lib):
    from chunkwise_gated_delta_local_amd import api
    assert status(prob(out_dtype=api.GDR_F32)) == 0
    assert status(prob(io_dtype=api.GDR_F32, out_dtype=api.GDR_BF16)) == 3
    assert status(prob(out_dtype=9)) == 3


def test_segmented_workspace_size(lib):
    """The segmented workspace is the production one plus, per segment, the
    local state, the transition and the entering state (fp32); shorter
    segments need more of it, and a negative segment length is an error."""
    from chunkwise_gated_delta_local_amd import api
    p = prob(seq_len=64 * 64)
    base = api.workspace_size(p)
    per_seg = 4 * p.num_v_heads * p.head_dim_qk * (2 * p.head_dim_v + p.head_dim_qk)
    s16 = api.workspace_size(p, segment_chunks=16)
    s4 = api.workspace_size(p, segment_chunks=4)
    assert base + per_seg * (64 // 16) <= s16 < s4
    assert s4 >= base + per_seg * (64 // 4)
    n = ctypes.c_size_t(0)
    assert lib.gdr_chunk_fwd_segmented_workspace_size(ctypes.byref(p), ctypes.c_int32(-1), ctypes.byref(n)) == 2


def test_segmented_automatic_choice_workspace(lib):
    """Automatic segments: a problem with few workgroups (here 2 sequences x 4
    value heads x 4 dv tiles = 32 < 64) gets room for up to 256 / 32 segments
    per sequence; one with 64 or more runs the serial pass and needs no segment
    states."""
    from chunkwise_gated_delta_local_amd import api
    small = prob(seq_len=64 * 256)
    per_seg = 4 * small.num_v_heads * small.head_dim_qk * (2 * small.head_dim_v + small.head_dim_qk)
    grid = small.num_seqs * small.num_v_heads * (small.head_dim_v // 16)
    assert grid < 64
    assert api.workspace_size(small, segment_chunks=0) >= (api.workspace_size(small)
                                                          + per_seg * small.num_seqs * (256 // grid))
    wide = prob(seq_len=64 * 256, Nk=32, Nv=32, dk=32, dv=32)
    per_seg_w = 4 * 32 * 32 * (2 * 32 + 32)
    assert api.workspace_size(wide, segment_chunks=0) < api.workspace_size(wide) + per_seg_w


def test_segmented_rejects_before_launch(lib):
    from chunkwise_gated_delta_local_amd import api
    if torch.cuda.is_available():
        pytest.skip("passes placeholder addresses; host-logic test for machines without a GPU")
    p = prob(seq_len=64 * 8)
    fake = ctypes.c_void_p(1 << 20)
    args = [ctypes.byref(p), fake, fake, fake, None, fake, ctypes.c_float(1.0), None, None, None, fake, None]
    assert lib.gdr_chunk_fwd_segmented(*args, ctypes.c_int32(-2), fake, ctypes.c_size_t(1 << 40), None, None) == 2
    assert lib.gdr_chunk_fwd_segmented(*args, ctypes.c_int32(1), None, ctypes.c_size_t(0), None, None) == 6
    serial_ws = api.workspace_size(p)           # enough for the serial pass, not for 1-chunk segments
    assert lib.gdr_chunk_fwd_segmented(*args, ctypes.c_int32(1), fake, ctypes.c_size_t(serial_ws), None, None) == 6


def test_backward_rejects_before_launch(lib):
    """gdr_chunk_bwd: missing gradient buffers, workspace or a misaligned
    pointer come back as status codes, with no device work."""
    from chunkwise_gated_delta_local_amd import api
    if torch.cuda.is_available():
        pytest.skip("passes placeholder addresses; host-logic test for machines without a GPU")
    p = prob()
    fake = ctypes.c_void_p(1 << 20)
    base = [ctypes.byref(p), fake, fake, fake, None, fake, ctypes.c_float(1.0), None, None, None]
    grads = [fake, None, fake, fake, fake, fake, None, None]       # d_o, dS_T, dq, dk, dv, dbeta, dg, dh0
    big = ctypes.c_size_t(1 << 40)
    assert lib.gdr_chunk_bwd(*base, *grads, None, ctypes.c_size_t(0), None, None) == 6
    bad = list(grads)
    bad[2] = None                                                   # dq missing
    assert lib.gdr_chunk_bwd(*base, *bad, fake, big, None, None) == 1
    bad = list(grads)
    bad[0] = None                                                   # d_o missing
    assert lib.gdr_chunk_bwd(*base, *bad, fake, big, None, None) == 1
    bad = list(grads)
    bad[4] = ctypes.c_void_p((1 << 20) + 4)                        # misaligned dv
    assert lib.gdr_chunk_bwd(*base, *bad, fake, big, None, None) == 2
    small = api.workspace_size(p)                                   # the forward's, not the backward's
    n = ctypes.c_size_t(0)
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0 and n.value > small
    assert lib.gdr_chunk_bwd(*base, *grads, fake, ctypes.c_size_t(small), None, None) == 6


def test_recurrent_rejects_before_launch(lib):
    """gdr_recurrent_fwd checks what every entry point checks: required
    pointers, and 16-byte alignment of every tensor it is given (outputs
    included), with no device work."""
    if torch.cuda.is_available():
        pytest.skip("passes placeholder addresses; host-logic test for machines without a GPU")
    p = prob()
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 4)
    # problem, q, k, v, g, beta, scale, S0, cu_dev, cu_host, l2norm, o, final_state, stream
    args = [ctypes.byref(p), fake, fake, fake, fake, fake, ctypes.c_float(1.0), fake, None, None, 0, fake, fake,
            None]
    for i in (1, 2, 3, 4, 5, 7, 11, 12):          # every tensor argument in turn
        bad = list(args)
        bad[i] = odd
        assert lib.gdr_recurrent_fwd(*bad) == 2, i
    bad = list(args)
    bad[11] = None                                 # o missing
    assert lib.gdr_recurrent_fwd(*bad) == 1


def test_noalloc_rejects_oversized_problem_before_any_device_call(lib):
    """gdr_chunk_fwd_noalloc refuses a problem whose workspace exceeds its
    per-GPU scratch with GDR_ERR_WORKSPACE, before touching a device."""
    from chunkwise_gated_delta_local_amd import api
    cap = lib.gdr_chunk_fwd_noalloc_max_workspace()
    assert cap == 256 << 20
    p = prob(batch=1, seq_len=65536, Nk=16, Nv=32, dk=128, dv=128, num_seqs=1)
    assert api.workspace_size(p) > cap
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: rejected first
    st = lib.gdr_chunk_fwd_noalloc(ctypes.byref(p), fake, fake, fake, None, fake, ctypes.c_float(1.0), None, None,
                                   None, fake, None, None)
    assert st == 6
    assert b"gdr_chunk_fwd_noalloc" in lib.gdr_last_error_message()
    # a problem that fits passes the size check (it then needs a device)
    small = prob(batch=2, seq_len=1000, Nk=4, Nv=4, dk=64, dv=64, num_seqs=2)
    assert api.workspace_size(small) <= cap
