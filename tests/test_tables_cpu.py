"""CPU models of the chunk-table and segment-table kernels and of the state
pass's chunk ranges, run on device offsets that disagree with the host's copy.

gdr.h promises that when cu_seqlens_dev and cu_seqlens_host differ the results
are unspecified but every kernel stays inside its buffers. The host sizes the
chunk table (nt_cap) and the segment table (nseg) from its own copy; the device
builds both tables from its copy. These models follow k_chunk_table,
k_segment_table and the range arithmetic of the fused state pass
(chunkwise_gated_delta_local_amd/csrc/gdr_kernels.hip) line for line in
integer arithmetic, and check that every chunk a segment walks has a length in
[0, 64] and a token range inside [0, Ttot), and that no segment crosses a
sequence boundary.
"""
import numpy as np
import pytest

C = 64


def chunk_table(cu, T_row, N, Ttot, cap):
    """Model of k_chunk_table: (chunk_seq, chunk_start, chunk_len, seq_first)."""
    chunk_seq = np.zeros(cap, np.int64)
    chunk_start = np.zeros(cap, np.int64)
    chunk_len = np.zeros(cap, np.int64)
    seq_first = np.zeros(N + 1, np.int64)

    def rng(n):
        s = cu[n] if cu is not None else n * T_row
        e = cu[n + 1] if cu is not None else (n + 1) * T_row
        s = min(max(s, 0), Ttot)
        e = min(max(e, s), Ttot)
        return s, e

    base = 0
    for n in range(N):
        s, e = rng(n)
        nch = (e - s + C - 1) // C
        seq_first[n] = min(base, cap)
        base += nch
    seq_first[N] = min(base, cap)
    total = min(base, cap)
    for c in range(total):
        n = max(i for i in range(N) if seq_first[i] <= c)   # last sequence whose first chunk is <= c
        s, e = rng(n)
        cs = s + (c - seq_first[n]) * C
        ce = min(cs + C, e)
        empty = not ce > cs
        chunk_seq[c] = n
        chunk_start[c] = 0 if empty else cs
        chunk_len[c] = 0 if empty else ce - cs
    return chunk_seq, chunk_start, chunk_len, seq_first


def segment_table(seq_first, N, seg_chunks, cap):
    """Model of k_segment_table: (seg_first [cap + 1], seq_seg [N + 1])."""
    end = seq_first[N]
    seg_first = np.full(cap + 1, end, np.int64)
    seq_seg = np.zeros(N + 1, np.int64)
    base = 0
    for n in range(N):
        f = seq_first[n]
        nch = seq_first[n + 1] - f
        nseg = (nch + seg_chunks - 1) // seg_chunks
        first = base
        seq_seg[n] = min(first, cap)
        for i in range(nseg):
            if first + i < cap:
                seg_first[first + i] = f + i * seg_chunks
        if first < cap and first + nseg >= cap:
            seg_first[cap] = f + nch
        base += nseg
    seq_seg[N] = min(base, cap)
    return seg_first, seq_seg


def walk(c0, c1, chunk_start, chunk_len):
    """The fused state pass's ranges for chunks c0..c1-1: (start, length) each."""
    seq_s = chunk_start[c0] if c0 < c1 else 0
    seq_e = chunk_start[c1 - 1] + chunk_len[c1 - 1] if c0 < c1 else 0
    out = []
    for c in range(c0, c1):
        s = seq_s + (c - c0) * C
        L = max(0, min(C, seq_e - s))
        out.append((s, L))
    return out


def host_counts(cu_host, T, N, seg_chunks):
    lens = [cu_host[n + 1] - cu_host[n] for n in range(N)]
    nt = sum((l + C - 1) // C for l in lens)
    nseg = sum(((l + C - 1) // C + seg_chunks - 1) // seg_chunks for l in lens)
    return T // C + N, nt, nseg   # nt_cap as make_plan sizes it


def check(cu_dev, cu_host, Ttot, seg_chunks):
    N = len(cu_host) - 1
    cap, _, nseg = host_counts(cu_host, Ttot, N, seg_chunks)
    chunk_seq, chunk_start, chunk_len, seq_first = chunk_table(cu_dev, 0, N, Ttot, cap)
    seg_first, seq_seg = segment_table(seq_first, N, seg_chunks, nseg)
    assert np.all(np.diff(seg_first) >= 0)
    assert seg_first[-1] <= cap
    for j in range(nseg):
        c0, c1 = seg_first[j], seg_first[j + 1]
        assert 0 <= c0 <= c1 <= cap
        if c0 < c1:
            assert len(set(chunk_seq[c0:c1])) == 1, ("segment crosses a sequence boundary", j)
        for s, L in walk(c0, c1, chunk_start, chunk_len):
            assert 0 <= L <= C
            if L > 0:
                assert 0 <= s and s + L <= Ttot, (j, s, L)
    for n in range(N):
        # the unsegmented pass walks seq_first[n] .. seq_first[n+1]
        for s, L in walk(seq_first[n], seq_first[n + 1], chunk_start, chunk_len):
            assert 0 <= L <= C and (L == 0 or 0 <= s and s + L <= Ttot)


def test_consistent_offsets_cover_every_token_once():
    cu = np.array([0, 5, 5, 200, 1000, 1001])
    cap, nt, nseg = host_counts(cu, 1001, 5, 2)
    chunk_seq, chunk_start, chunk_len, seq_first = chunk_table(cu, 0, 5, 1001, cap)
    covered = np.zeros(1001, int)
    for c in range(nt):
        covered[chunk_start[c]:chunk_start[c] + chunk_len[c]] += 1
    assert np.all(covered == 1)
    check(cu, cu, 1001, 2)


@pytest.mark.parametrize("seg_chunks", [1, 2, 3, 7])
@pytest.mark.parametrize("case", [
    # (device offsets, host offsets, Ttot): the device copy has more chunks than the host counted
    ([0, 1000, 1000], [0, 10, 1000], 1000),
    ([0, 1, 999, 1000], [0, 500, 501, 1000], 1000),
    # decreasing and out-of-range device offsets
    ([0, 900, 100, 1000], [0, 300, 600, 1000], 1000),
    ([0, -50, 5000, 1000], [0, 400, 700, 1000], 1000),
    # one long sequence on the device, many short ones on the host
    ([0, 4096, 4096, 4096, 4096], [0, 1, 2, 3, 4096], 4096),
])
def test_mismatched_offsets_stay_in_bounds(case, seg_chunks):
    cu_dev, cu_host, Ttot = case
    check(np.array(cu_dev), np.array(cu_host), Ttot, seg_chunks)


def test_random_mismatches():
    rng = np.random.default_rng(3)
    for _ in range(200):
        N = int(rng.integers(1, 6))
        Ttot = int(rng.integers(1, 3000))
        host = np.sort(rng.integers(0, Ttot + 1, N + 1))
        host[0], host[-1] = 0, Ttot
        dev = rng.integers(-100, Ttot + 100, N + 1)
        check(dev, host, Ttot, int(rng.integers(1, 5)))
