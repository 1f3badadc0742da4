"""Host check of the matrix-state kernels' addressing (csrc/wkv_mat.hip).

The element offsets each thread of mat_forward_kernel and mat_step_kernel
forms are recomputed here from the same formulas, for every workgroup and
thread of small launches, and checked against the arrays' bounds -- including
T = 0, where the forward must not load at all (its token clamp needs a token),
and the chunks past the last one that its 4-deep prefetch ring loads.
CPU only.
"""
import numpy as np
import pytest

N = 64        # head dimension
CT = 16       # tokens per chunk
PREFETCH = 4  # chunks in the register ring


def forward_offsets(B, T, H):
    """(loads, stores, state) element offsets of mat_forward_kernel: 512
    threads per (batch row, head); waves 4..7 load (producers), waves 0..3
    store y and hold the state (consumers)."""
    C = H * N
    loads, stores, state = [], [], []
    nch = (T + CT - 1) // CT
    for blk in range(B * H):
        bb, h = divmod(blk, H)
        row0 = bb * T
        for thr in range(512):
            wave, lane = divmod(thr, 64)
            producer = wave >= 4
            tt, i0 = lane & 15, 4 * (4 * (wave & 3) + (lane >> 4))
            g, nn = lane >> 4, lane & 15
            jcol = 16 * (wave & 3) + nn
            if producer:
                if nch == 0:
                    continue
                e0 = row0 * C + h * N + i0
                q0 = -PREFETCH
                while q0 <= nch:
                    for p in range(PREFETCH):
                        t = (q0 + p + PREFETCH) * CT + tt
                        t = t if t < T else T - 1
                        loads.extend(e0 + t * C + q for q in range(4))
                    q0 += PREFETCH
                continue
            for b in range(4):
                for r in range(4):
                    state.append((bb * H + h) * N * N + (16 * b + 4 * g + r) * N + jcol)
            for ch in range(nch):
                t0 = ch * CT
                n = max(0, min(CT, T - t0))
                ct = wave * 64 + lane   # chunked form's output: the y tile in whole rows
                row, cg = ct >> 4, (ct & 15) * 4
                if row < n:
                    stores.extend((row0 + t0 + row) * C + h * N + cg + q for q in range(4))
                for t in range(n):    # token-by-token form: its inputs read from global memory
                    e = (row0 + t0 + t) * C + h * N
                    stores.append(e + jcol)
                    loads.append(e + jcol)
                    loads.extend(e + 16 * b + 4 * g + q for b in range(4) for q in range(4))
    return np.array(loads, dtype=np.int64), np.array(stores, dtype=np.int64), np.array(state)


@pytest.mark.parametrize("B,T,H", [(2, 0, 3), (1, 1, 1), (1, 15, 2), (2, 16, 1), (1, 17, 1),
                                   (2, 53, 2), (1, 100, 1), (1, 129, 1)])
def test_forward_addresses_stay_in_bounds(B, T, H):
    loads, stores, state = forward_offsets(B, T, H)
    n_io = B * T * H * N
    if T == 0:
        assert loads.size == 0 and stores.size == 0
        assert state.min() >= 0 and state.max() < B * H * N * N
        return
    else:
        assert loads.min() >= 0 and loads.max() < n_io
        assert stores.min() >= 0 and stores.max() < n_io
        # every output element is written
        assert np.array_equal(np.unique(stores), np.arange(n_io))
    assert state.min() >= 0 and state.max() < B * H * N * N
    assert np.array_equal(np.unique(state), np.arange(B * H * N * N))


@pytest.mark.parametrize("L,S,H", [(1, 1, 1), (2, 3, 2), (1, 1, 5)])
def test_step_addresses_stay_in_bounds(L, S, H):
    """mat_step_kernel: wave = head; lane (rg, cq) reads and writes columns
    4cq .. 4cq+3 of rows 4m + rg of the head's state; the key-channel table is
    read with one element per lane; y is written by the lanes of row group 0."""
    C = H * N
    heads = L * S * H
    io_loads, y_stores, st = [], [], []
    for blk in range((heads + 3) // 4):
        for thr in range(256):
            head = blk * 4 + thr // 64
            lane = thr & 63
            if head >= heads:
                continue
            row, h = divmod(head, H)
            e0 = row * C + h * N
            io_loads.append(e0 + lane)                          # z, k, r of key channel lane
            rg, cq = lane >> 4, lane & 15
            io_loads.extend(e0 + 4 * cq + q for q in range(4))  # v of the lane's columns
            sb = head * N * N + rg * N + 4 * cq
            st.extend(sb + m * 4 * N + q for m in range(16) for q in range(4))
            if rg == 0:
                y_stores.extend(e0 + 4 * cq + q for q in range(4))
    io_loads, y_stores, st = np.array(io_loads), np.array(y_stores), np.array(st)
    assert io_loads.min() >= 0 and io_loads.max() < L * S * C
    assert np.array_equal(np.unique(y_stores), np.arange(L * S * C))
    assert np.array_equal(np.unique(st), np.arange(heads * N * N))
    assert st.size == heads * N * N            # each state element once
