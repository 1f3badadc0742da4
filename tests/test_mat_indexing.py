"""Host check of the matrix-state kernels' addressing (csrc/wkv_mat.hip).

The element offsets each thread of mat_forward_tokens_kernel,
mat_forward_ring_kernel and mat_step_kernel
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


def paired_task(bid, n):
    """Workgroup -> (batch row, head) task of the forward kernels: heads 2j,
    2j + 1 on workgroups j, j + n/2 (plain order for an odd count)."""
    if n % 2:
        return bid
    half = n // 2
    return 2 * bid if bid < half else 2 * (bid - half) + 1


@pytest.mark.parametrize("n", [1, 2, 3, 7, 8, 64, 511, 512])
def test_paired_task_is_a_bijection(n):
    tasks = [paired_task(b, n) for b in range(n)]
    assert sorted(tasks) == list(range(n))
    if n % 2 == 0:
        # the two halves of each 256-byte row piece are half a grid apart
        for j in range(n // 2):
            assert (tasks[j], tasks[j + n // 2]) == (2 * j, 2 * j + 1)


def forward_offsets(B, T, H):
    """(loads, stores, state) element offsets of mat_forward_tokens_kernel:
    512 threads per (batch row, head); waves 4..7 load (producers), waves 0..3
    store y and hold the state (consumers)."""
    C = H * N
    loads, stores, state = [], [], []
    nch = (T + CT - 1) // CT
    for blk in range(B * H):
        bb, h = divmod(paired_task(blk, B * H), H)
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
                for t in range(n):    # y of column jcol, token by token
                    if g == 0:
                        stores.append((row0 + t0 + t) * C + h * N + jcol)
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


def ring_offsets(B, T, H, per_token_z=True, strict_size=True):
    """Byte offsets of mat_forward_ring_kernel (bf16): the producer loads of
    every (batch row, head), with the buffer descriptor's size check applied
    (strict_size: an access is dropped unless it ends within the size; else
    only when it starts at or past it), the operand-tile writes, and the y
    stores of the chunked form.  Returns (loads, y_stores, tile_writes)."""
    C = H * N
    row_bytes = 2 * C
    nch = (T + CT - 1) // CT
    loads, ystores, tiles = [], [], []
    for blk in range(B * H):
        bb, h = divmod(paired_task(blk, B * H), H)
        row0 = bb * T
        for p in range(4):                       # producer wave p (waves 4..7)
            chunks = []
            q = p
            chunks.append(q)                     # the first load, before the loop
            while q < nch:
                chunks.append(q + 4)             # prefetch into the other set
                if q + 4 >= nch:
                    break
                chunks.append(q + 8)
                q += 8
            for q in chunks:
                inside = q < nch
                t0 = q * CT if inside else 0
                rows = min(CT, T - t0) if inside else 0
                base = ((row0 + t0) * C + h * N) * 2
                size = None if rows == CT else (rows * row_bytes - h * N * 2 if rows > 0 else 0)
                for lane in range(64):
                    g, n = lane >> 4, lane & 15
                    for j in range(4):
                        off = (4 * g + j) * row_bytes + 8 * n
                        if size is not None:
                            dropped = off + 8 > size if strict_size else off >= size
                            if dropped:
                                continue
                        loads.append(((base + off) // 2, bb, h))
            for q in range(p, nch, 4):
                for lane in range(64):
                    g, n = lane >> 4, lane & 15
                    for j in range(4):
                        tiles.append(("rq", 4 * g + j, 4 * n))
                    for c in range(4):
                        tiles.append(("kdt", 4 * n + c, 4 * g))
        for q in range(nch):
            live = min(CT, T - q * CT)
            for lane in range(64):
                g, nn = lane >> 4, lane & 15
                for i in range(4):
                    row = 4 * i + g
                    if row < live:
                        e = (row0 + q * CT + row) * C + h * N + 4 * nn
                        ystores.extend(e + c for c in range(4))
    return np.array(loads, dtype=np.int64).reshape(-1, 3), np.array(ystores, dtype=np.int64), tiles


@pytest.mark.parametrize("strict", [True, False])
@pytest.mark.parametrize("B,T,H", [(2, 0, 3), (1, 1, 1), (1, 5, 2), (2, 16, 1), (1, 17, 3),
                                   (2, 53, 2), (1, 100, 1), (2, 129, 2)])
def test_ring_addresses_stay_in_bounds(B, T, H, strict):
    loads, ystores, tiles = ring_offsets(B, T, H, strict_size=strict)
    n_io = B * T * H * N
    if T == 0:
        assert loads.size == 0 and ystores.size == 0
        return
    # every load lands on the workgroup's own batch row and head (so never on
    # a token past T), and every element is loaded
    el, bb, h = loads[:, 0], loads[:, 1], loads[:, 2]
    assert el.min() >= 0 and el.max() + 3 < n_io
    C = H * N
    assert np.array_equal(el // C // T, bb)
    assert np.array_equal((el % C) // N, h)
    assert np.array_equal(np.unique(el // 4 * 4), np.arange(0, n_io, 4))
    # each y element written exactly once
    assert ystores.size == n_io
    assert np.array_equal(np.sort(ystores), np.arange(n_io))
    for name, r, c in tiles:
        if name == "rq":
            assert 0 <= r < CT and 0 <= c and c + 3 < N
        else:
            assert 0 <= r < N and 0 <= c and c + 3 < CT
