"""The C-ABI libraries load and export what include/*.h declares; host-side
argument validation.  CPU only: no call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import linear_attention_rnn_forward_amd as wkv
import synth.device

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECL = re.compile(r"^\s*(?:const\s+)?(?:int|size_t|char|void)\s*\*?\s*(\w+)\s*\(", re.M)


def _declared(header):
    with open(os.path.join(ROOT, "include", header)) as f:
        return sorted(set(DECL.findall(f.read())))


@pytest.mark.parametrize("header,libpath", [("wkv.h", wkv.LIB_PATH),
                                            ("wkv_synth.h", synth.device.LIB_PATH)])
def test_every_declared_symbol_is_exported(header, libpath):
    names = _declared(header)
    assert names, header
    lib = ctypes.CDLL(libpath)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"{os.path.basename(libpath)} lacks {missing}"


def test_header_lists_the_boundary_calls():
    names = _declared("wkv.h")
    for n in ("wkv_forward", "wkv_step", "wkv_token_shift", "wkv_forward_workspace_size",
              "wkv_forward_gated", "wkv_step_gated", "wkv_backward", "wkv_backward_workspace_size",
              "wkv_status_string", "wkv_last_error", "wkv_mat_forward", "wkv_mat_forward_path",
              "wkv_mat_step", "wkv_bounded_wait_failures", "wkv_forward_auto_path",
              "wkv_forward_save", "wkv_backward_saved", "wkv_saved_states_bytes",
              "wkv_backward_saved_workspace_size"):
        assert n in names


def test_abi_version_and_status_strings():
    L = wkv.lib()
    assert L.wkv_abi_version() == 107 == wkv.ABI_VERSION
    for code in range(0, -9, -1):
        assert L.wkv_status_string(code).decode()
    assert L.wkv_status_string(-100).decode() == "unknown status"


def test_binding_refuses_another_abi_version(monkeypatch):
    """Buffer layouts (the saved states among them) change with the ABI
    version, so the binding will not drive a library built for another."""
    monkeypatch.setattr(wkv, "_lib", None)
    monkeypatch.setattr(wkv, "ABI_VERSION", wkv.ABI_VERSION + 1)
    with pytest.raises(RuntimeError, match="ABI version"):
        wkv.lib()
    monkeypatch.undo()
    assert wkv.lib().wkv_abi_version() == wkv.ABI_VERSION


P = ctypes.c_void_p


G = 1 << 30   # fake device addresses, far enough apart not to overlap


def _fwd(path=0, B=1, T=8, C=64, dtype=0, w=1 * G, u=2 * G, k=3 * G, v=4 * G, y=5 * G, a_in=None, b_in=None, p_in=None, a_out=None, b_out=None, p_out=None,
         ws=None, ws_bytes=0):
    L = wkv.lib()
    return L.wkv_forward_path(B, T, C, dtype, path, P(w), P(u), P(k), P(v), P(y), P(a_in),
                              P(b_in), P(p_in), P(a_out), P(b_out), P(p_out), P(ws), ws_bytes,
                              None)


def test_forward_rejects_bad_arguments():
    L = wkv.lib()
    assert _fwd(dtype=7) == -3
    assert _fwd(B=0) == -2 and _fwd(C=0) == -2 and _fwd(T=-1) == -2
    assert _fwd(B=1 << 40, T=1 << 40) == -2
    # a block of 32 token rows must stay within 32-bit byte offsets
    for dtype, es in ((0, 4), (1, 2)):
        c_max = (4294967295 - 512) // (33 * es)
        assert _fwd(C=c_max + 1, T=1, dtype=dtype) == -2
        assert b"32-bit offsets" in L.wkv_last_error()
    assert _fwd(path=9) == -8
    assert _fwd(k=None) == -1 and _fwd(w=None) == -1
    assert _fwd(a_in=6 * G) == -1          # state in: all or none
    assert _fwd(a_out=6 * G, b_out=7 * G) == -1
    # y overlapping k
    assert _fwd(y=3 * G + 16) == -5
    assert b"y overlaps k" in L.wkv_last_error()
    # state out overlapping a different state input
    st = dict(a_in=8 * G, b_in=9 * G, p_in=10 * G)
    assert _fwd(**st, a_out=9 * G, b_out=11 * G, p_out=12 * G) == -5
    assert _fwd(**st, a_out=8 * G + 4, b_out=11 * G, p_out=12 * G) == -5   # partial overlap
    # chunked path without workspace
    assert _fwd(path=2, T=1024) == -4
    need = L.wkv_forward_workspace_size_path(1, 1024, 64, 0, 2)
    assert need > 0
    assert _fwd(path=2, T=1024, ws=13 * G, ws_bytes=need - 1) == -4
    assert _fwd(path=2, T=1024, ws=13 * G + 8, ws_bytes=need) == -4   # misaligned


def test_step_and_shift_reject_bad_arguments():
    L = wkv.lib()
    args = [P(G * (i + 1)) for i in range(11)]
    assert L.wkv_step(0, 1, 1, 0, *args, None) == -2
    assert L.wkv_step(1, 1, 4, 5, *args, None) == -3
    nul = list(args)
    nul[3] = P(None)
    assert L.wkv_step(1, 1, 4, 0, *nul, None) == -1
    # y (index 4) equal to k (index 2)
    al = list(args)
    al[4] = al[2]
    assert L.wkv_step(1, 1, 4, 0, *al, None) == -5
    sa = [P(G * (i + 1)) for i in range(9)]
    assert L.wkv_token_shift(0, 4, 4, 0, *sa, None) == -2
    bad = list(sa)
    bad[5] = sa[0]   # xr == x
    assert L.wkv_token_shift(1, 4, 4, 0, *bad, None) == -5


def test_workspace_sizes():
    L = wkv.lib()
    # serial path and T = 0 need none; the chunked path needs flags + partial states
    assert L.wkv_forward_workspace_size_path(4, 100, 64, 0, 1) == 0
    assert L.wkv_forward_workspace_size_path(4, 0, 64, 0, 2) == 0
    n = L.wkv_forward_workspace_size_path(1, 65536, 4096, 0, 2)
    assert 256 < n < 128 << 20
    assert L.wkv_forward_workspace_size_path(0, 10, 10, 0, 2) == 0


def test_chunked_workspace_covers_both_tile_widths():
    # B=8 T=1024 C=768 fp32 takes 16-wave tiles on a 256-CU part (192 tiles);
    # the size query plans for 8-wave tiles (384), the larger workspace:
    # 256 bytes of counters, a 256-byte-rounded 8-byte flag per tile and two
    # 4-field fp32 descriptors of 64 channels per tile
    L = wkv.lib()
    tiles = 8 * (768 // 64) * (1024 // 256)
    flags = (tiles * 8 + 255) // 256 * 256
    assert L.wkv_forward_workspace_size_path(8, 1024, 768, 0, 2) == 256 + flags + tiles * 2 * 4 * 64 * 4


def test_auto_path_query():
    # without a visible device the library assumes 256 compute units (MI355X)
    assert wkv.auto_path(16, 4096, 2048, wkv.BF16) == "chained"   # 256 column groups
    assert wkv.auto_path(1, 65536, 4096, wkv.F32) == "chunked"    # 64 column groups
    assert wkv.auto_path(256, 512, 4096, wkv.F32) == "serial"     # 16384 column groups
    assert wkv.auto_path(1, 16, 64, wkv.F32) == "serial"          # a single block
    L = wkv.lib()
    assert L.wkv_forward_auto_path(0, 8, 8, 0) == -2
    assert L.wkv_forward_auto_path(1, 8, 8, 5) == -3


def _fwd_gated(path=0, B=1, T=8, C=64, dtype=0, w=1 * G, u=2 * G, k=3 * G, v=4 * G, r=6 * G, o=5 * G,
               a_in=None, b_in=None, p_in=None, a_out=None, b_out=None, p_out=None):
    L = wkv.lib()
    return L.wkv_forward_gated(B, T, C, dtype, path, P(w), P(u), P(k), P(v), P(r), P(o), P(a_in),
                               P(b_in), P(p_in), P(a_out), P(b_out), P(p_out), None, 0, None)


def test_forward_gated_rejects_bad_arguments():
    """r is required (T > 0) and the output may not overlap it; the plain
    checks apply unchanged."""
    assert _fwd_gated(r=None) == -1            # WKV_ERR_NULL
    assert _fwd_gated(r=5 * G) == -5           # o overlaps r
    assert _fwd_gated(r=5 * G + 64) == -5      # partial overlap
    assert _fwd_gated(dtype=7) == -3
    assert _fwd_gated(B=0) == -2
    assert _fwd_gated(path=9) == -8
    assert _fwd_gated(a_out=7 * G, b_out=8 * G, p_out=6 * G) == -5   # state output overlaps r
    # T = 0 needs no r
    L = wkv.lib()
    assert L.wkv_forward_gated(1, 0, 64, 0, 0, P(G), P(2 * G), None, None, None, None, None, None,
                               None, None, None, None, None, 0, None) == 0


def test_step_gated_rejects_bad_arguments():
    L = wkv.lib()
    n = [P(i * G) for i in range(1, 13)]   # w u k v r y a_in b_in p_in a_out b_out p_out

    def call(**over):
        args = dict(zip("w u k v r y ai bi pi ao bo po".split(), n))
        args.update({k2: P(v2) if v2 is not None else None for k2, v2 in over.items()})
        return L.wkv_step_gated(2, 3, 64, 0, args["w"], args["u"], args["k"], args["v"], args["r"],
                                args["y"], args["ai"], args["bi"], args["pi"], args["ao"], args["bo"],
                                args["po"], None)

    assert call(r=None) == -1
    assert call(r=6 * G) == -5        # y (6 G) overlaps r
    assert call(ao=5 * G) == -5       # a_out overlaps r


def test_session_blob_size():
    """Header plus a, b, p (fp32) and the shifted tokens: for the pages' 7B
    configuration (32 layers, 4096 channels, two token-shifting sub-blocks,
    bf16 shifts) that is 64 + 32*4096*(12 + 2*2) bytes."""
    L = wkv.lib()
    assert L.wkv_session_bytes(32, 4096, 1, 2) == 64 + 32 * 4096 * 16
    assert L.wkv_session_bytes(2, 3, 0, 0) == 64 + 2 * 3 * 12
    assert L.wkv_session_bytes(0, 8, 0, 0) == 0
    assert L.wkv_session_bytes(2, 8, 5, 0) == 0
    assert L.wkv_session_bytes(2, 8, 0, 9) == 0


def test_session_load_checks_the_header_first():
    """A wrong magic, version, shape or a short blob is refused before any
    copy is enqueued (the device pointers here are never touched)."""
    import struct
    L = wkv.lib()
    Ln, S, C, dt, ns = 2, 3, 8, 0, 1
    n = L.wkv_session_bytes(Ln, C, dt, ns)
    good = struct.pack("<IIqqii", 0x53564B57, 1, Ln, C, dt, ns).ljust(64, b"\0") + bytes(n - 64)
    fake = [P(i * G) for i in range(1, 5)]
    shifts = (ctypes.c_void_p * 1)(4 * G)

    def load(blob, **kw):
        args = dict(L=Ln, S=S, C=C, dt=dt, seq=1, ns=ns)
        args.update(kw)
        buf = ctypes.create_string_buffer(blob, len(blob))
        return L.wkv_session_load(args["L"], args["S"], args["C"], args["dt"], args["seq"], buf,
                                  len(blob), fake[0], fake[1], fake[2], shifts, args["ns"], None)

    bad_magic = b"XXXX" + good[4:]
    bad_version = good[:4] + struct.pack("<I", 7) + good[8:]
    assert load(bad_magic) == -8
    assert load(bad_version) == -7
    assert load(good, C=16) == -8          # saved with another C
    assert load(good, ns=0) == -8          # saved with another n_shift
    assert load(good[:100]) == -8          # truncated
    assert load(good[:10]) == -8           # shorter than the header
    assert load(good, seq=3) == -8         # seq out of range
    assert load(good, S=0) == -2
    load(bad_magic)
    assert b"magic" in L.wkv_last_error()


def test_session_save_checks_arguments():
    L = wkv.lib()
    buf = ctypes.create_string_buffer(10)
    # blob too small: refused before any copy
    assert L.wkv_session_save(2, 3, 8, 0, 0, P(G), P(2 * G), P(3 * G), None, 0, buf, 10, None) == -8
    assert L.wkv_session_save(2, 3, 8, 0, 0, None, P(2 * G), P(3 * G), None, 0, buf, 10, None) == -1
    assert L.wkv_session_save(2, 3, 8, 0, 5, P(G), P(2 * G), P(3 * G), None, 0, buf, 10, None) == -8
    assert L.wkv_session_save(2, 3, 8, 0, 0, P(G), P(2 * G), P(3 * G), None, 1, buf, 10, None) == -1


def test_backward_workspace_size():
    """The forward state before every 16-token sub-chunk (2 fp32 per column)
    plus per-column gw, gu partials, each section rounded up to 256 bytes."""
    L = wkv.lib()
    assert L.wkv_backward_workspace_size(2, 3, 64) == 1024 + 2 * 512
    assert L.wkv_backward_workspace_size(2, 17, 64) == 2 * 1024 + 2 * 512
    assert L.wkv_backward_workspace_size(16, 4096, 2048) == 16 * 2048 * 256 * 8 + 2 * 16 * 2048 * 4
    assert L.wkv_backward_workspace_size(1, 1, 1) == 3 * 256
    assert L.wkv_backward_workspace_size(0, 8, 8) == 0
    assert L.wkv_backward_workspace_size(1 << 40, 1 << 40, 8) == 0


def test_backward_rejects_bad_arguments():
    L = wkv.lib()
    B, T, C = 2, 3, 64
    need = L.wkv_backward_workspace_size(B, T, C)

    def call(dtype=0, B=B, T=T, C=C, ws=20 * G, ws_bytes=need, **over):
        a = dict(w=1, u=2, k=3, v=4, gy=5, gk=6, gv=7, gw=8, gu=9)
        a.update(over)
        ptr = {n: (P(int(x * G)) if x is not None else None) for n, x in a.items()}
        return L.wkv_backward(B, T, C, dtype, ptr["w"], ptr["u"], ptr["k"], ptr["v"], ptr["gy"],
                              ptr["gk"], ptr["gv"], ptr["gw"], ptr["gu"], P(ws) if ws else None,
                              ws_bytes, None)

    assert call(dtype=5) == -3
    assert call(B=0) == -2 and call(C=0) == -2 and call(T=-1) == -2
    assert call(B=1 << 40, T=1 << 40) == -2
    assert call(gw=None) == -1 and call(u=None) == -1
    assert call(gy=None) == -1 and call(gk=None) == -1
    assert call(gk=4) == -5                        # gk on v
    assert b"gk overlaps v" in L.wkv_last_error()
    assert call(gu=8) == -5                        # gu on gw
    assert call(ws=None) == -4
    assert call(ws_bytes=need - 1) == -4
    assert call(ws=20 * G + 16) == -4              # misaligned
    assert call(ws=6 * G) == -5                    # workspace on gk
    assert call(C=1 << 26) == -2                   # sub-chunk offsets beyond 32 bits


def test_saved_state_sizes():
    """[B][ceil(T/16)][2][C] fp32 states; the saved backward's workspace is
    only the per-column partials."""
    L = wkv.lib()
    assert L.wkv_saved_states_bytes(2, 3, 64) == 2 * 1 * 2 * 64 * 4
    assert L.wkv_saved_states_bytes(2, 17, 64) == 2 * 2 * 2 * 64 * 4
    assert L.wkv_saved_states_bytes(16, 4096, 2048) == 16 * 256 * 2 * 2048 * 4
    assert L.wkv_saved_states_bytes(1, 0, 8) == 0
    assert L.wkv_saved_states_bytes(0, 8, 8) == 0
    assert L.wkv_backward_saved_workspace_size(2, 64) == 2 * 512
    assert L.wkv_backward_saved_workspace_size(16, 2048) == 2 * 16 * 2048 * 4
    assert L.wkv_backward_saved_workspace_size(0, 8) == 0
    assert wkv.saved_states_shape(2, 17, 64) == (2, 2, 2, 64)


def test_forward_save_rejects_bad_arguments():
    L = wkv.lib()

    def call(dtype=0, B=2, T=33, C=64, **over):
        a = dict(w=1, u=2, k=3, v=4, y=5, states=6)
        a.update(over)
        ptr = {n: (P(int(x * G)) if x is not None else None) for n, x in a.items()}
        return L.wkv_forward_save(B, T, C, dtype, ptr["w"], ptr["u"], ptr["k"], ptr["v"], ptr["y"],
                                  ptr["states"], None)

    assert call(dtype=5) == -3
    assert call(B=0) == -2 and call(T=-1) == -2
    assert call(states=None) == -1
    assert call(states=3) == -5                   # states on k
    assert b"states overlaps k" in L.wkv_last_error()
    assert call(states=5) == -5                   # states on y
    assert call(states=6 + 4 / G) == -8            # misaligned (4 bytes off)


def test_backward_saved_rejects_bad_arguments():
    L = wkv.lib()
    B, T, C = 2, 33, 64
    need = L.wkv_backward_saved_workspace_size(B, C)

    def call(ws=20 * G, ws_bytes=need, **over):
        a = dict(w=1, u=2, k=3, v=4, gy=5, states=10, gk=6, gv=7, gw=8, gu=9)
        a.update(over)
        ptr = {n: (P(int(x * G)) if x is not None else None) for n, x in a.items()}
        return L.wkv_backward_saved(B, T, C, 0, ptr["w"], ptr["u"], ptr["k"], ptr["v"], ptr["gy"],
                                    ptr["states"], ptr["gk"], ptr["gv"], ptr["gw"], ptr["gu"],
                                    P(ws) if ws else None, ws_bytes, None)

    assert call(states=None) == -1
    assert call(gk=10) == -5                      # gk on the states
    assert b"gk overlaps states" in L.wkv_last_error()
    assert call(ws=10 * G) == -5                  # workspace on the states
    assert call(ws_bytes=need - 1) == -4
    assert call(states=10 + 4 / G) == -8           # misaligned (4 bytes off)


# ---------------------------------------------------------------------------
# matrix-valued state calls: validation happens before any launch
# ---------------------------------------------------------------------------

def _mat_fwd(path=0, B=1, T=8, H=2, dtype=1, r=1 * G, k=2 * G, v=3 * G, z=4 * G, z_mode=1,
             s_in=None, s_out=None, y=5 * G):
    return wkv.lib().wkv_mat_forward_path(B, T, H, dtype, path, P(r), P(k), P(v), P(z), z_mode,
                                          P(s_in), P(s_out), P(y), None)


def _mat_step(L=2, S=3, H=2, dtype=0, r=1 * G, k=2 * G, v=3 * G, z=4 * G, z_mode=0,
              s_in=6 * G, s_out=7 * G, y=5 * G):
    return wkv.lib().wkv_mat_step(L, S, H, dtype, P(r), P(k), P(v), P(z), z_mode, P(s_in),
                                  P(s_out), P(y), None)


def test_mat_forward_rejects_bad_arguments():
    L = wkv.lib()
    assert _mat_fwd(dtype=5) == -3
    assert _mat_fwd(B=0) == -2 and _mat_fwd(H=0) == -2 and _mat_fwd(T=-1) == -2
    assert _mat_fwd(B=1 << 40, T=1 << 30) == -2
    assert _mat_fwd(path=7) == -8
    assert _mat_fwd(z_mode=3) == -8
    assert _mat_fwd(path=1, dtype=0) == -7          # chunked form: bf16 storage only
    assert _mat_fwd(r=None) == -1 and _mat_fwd(z=None) == -1 and _mat_fwd(y=None) == -1
    assert _mat_fwd(k=2 * G + 2) == -8             # misaligned
    assert _mat_fwd(y=3 * G + 64) == -5            # y overlaps v
    assert b"y overlaps v" in L.wkv_last_error()
    # the state out may be the state in, but may not overlap another input
    assert _mat_fwd(s_in=6 * G, s_out=4 * G) == -5
    assert _mat_fwd(s_in=6 * G, s_out=6 * G + 256) == -5
    # T = 0 with no state wanted: nothing to do, nothing launched
    assert _mat_fwd(T=0, r=None, k=None, v=None, z=None, y=None) == 0


def test_mat_step_rejects_bad_arguments():
    L = wkv.lib()
    assert _mat_step(dtype=2) == -3
    assert _mat_step(L=0) == -2 and _mat_step(S=0) == -2 and _mat_step(H=0) == -2
    assert _mat_step(s_in=None) == -1 and _mat_step(s_out=None) == -1
    assert _mat_step(v=None) == -1
    assert _mat_step(z_mode=2) == -8
    assert _mat_step(dtype=0, r=1 * G + 8) == -8   # fp32 needs 16-byte alignment
    assert _mat_step(y=2 * G) == -5                # y is k
    assert _mat_step(s_out=3 * G) == -5            # state out overlaps v
    assert b"s_out overlaps v" in L.wkv_last_error()


def test_noalloc_rejects_sizes_beyond_its_scratch():
    L = wkv.lib()
    P_ = ctypes.c_void_p
    def call(B, T, C, dtype=0):
        return L.wkv_forward_noalloc(B, T, C, dtype, P_(1 * G), P_(2 * G), P_(3 * G), P_(4 * G),
                                     P_(5 * G), None, None, None, None, None, None, None)
    # long context at 16x the channels: its chunked workspace is far beyond 40 MiB
    assert L.wkv_forward_workspace_size(1, 1 << 20, 8192, 0) > 40 << 20
    assert call(1, 1 << 20, 8192) == -4
    assert b"scratch" in L.wkv_last_error()
    # invalid sizes are reported as such
    assert call(0, 8, 8) == -2
