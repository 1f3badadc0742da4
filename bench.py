#!/usr/bin/env python3
"""Throughput of the WKV operator on one MI355X.

Default workload: wkv_forward over B=16, T=4096, C=2048 with bf16 k/v/y and
fp32 w/u/state (the configuration the bandwidth target is stated for).  A
step is one wkv_forward call over that batch; inputs are synthetic (seeded,
shaped like the pages' setting) and already resident in HBM.

Prints one JSON line with tokens*channels/s, the dominant kernel's achieved
HBM bandwidth against the 8 TB/s peak (algorithmic bytes over the kernel's
average duration, timed with HIP events on the launch stream), and the fp64
CPU oracle timed on the same workload on the host cores.

Other workloads (--workload): tiny, small_lm, long_ctx (wkv_forward),
bf16_main_gated (the default workload through wkv_forward_gated, the
receptance gate fused), bf16_main_backward (wkv_backward over the default
workload's shape; a step is its two launches), bf16_main_backward_saved
(wkv_backward_saved from wkv_forward_save's states, made before the timed
region; the line also reports what saving them adds to the forward), decode (wkv_step over [32,256,4096] fp32),
token_shift (bf16, B=16 T=4096 C=2048), mat_main / mat_eagle (the
matrix-valued-state operator of RWKV-6 Finch / RWKV-5 Eagle, wkv_mat_forward
over B=16 T=4096 and 32 heads of 64, bf16), mat_decode (wkv_mat_step over
32 layers x 64 sequences x 64 heads, fp32).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "WKV forward tokens·channels/s and achieved HBM GB/s (% of peak) at 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# The sources that define each workload's kernels and their launch geometry
# (the C ABI layer only validates and dispatches).
_COMMON_SOURCES = ["wkv_device.h", "wkv_internal.h"]
_FORWARD_SOURCES = ["wkv_forward.hip"] + _COMMON_SOURCES
KERNEL_SOURCES = {
    "tiny": _FORWARD_SOURCES, "small_lm": _FORWARD_SOURCES, "bf16_main": _FORWARD_SOURCES,
    "bf16_main_gated": _FORWARD_SOURCES, "long_ctx": _FORWARD_SOURCES,
    "bf16_main_backward": ["wkv_backward.hip"] + _COMMON_SOURCES,
    "bf16_main_backward_saved": ["wkv_backward.hip"] + _COMMON_SOURCES,
    "decode": ["wkv_step.hip"] + _COMMON_SOURCES,
    "token_shift": ["wkv_token_shift.hip"] + _COMMON_SOURCES,
    "mat_main": ["wkv_mat.hip"] + _COMMON_SOURCES, "mat_eagle": ["wkv_mat.hip"] + _COMMON_SOURCES,
    "mat_decode": ["wkv_mat.hip"] + _COMMON_SOURCES,
}


def _code_only(text: str) -> str:
    """C++ source without its comments and blank lines (comments do not
    change the compiled kernels; the sources hold no comment markers inside
    string literals)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def kernel_source_hash(workload: str) -> str:
    """Hash of the code (comments left out) of the kernel sources of
    `workload` (every source when unknown)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_rnn_forward_amd", "csrc")
    names = KERNEL_SOURCES.get(workload) or sorted(os.listdir(csrc))
    for name in sorted(names):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("source_hash") != kernel_source_hash(workload):
        return None
    return entry.get("traffic_bytes_per_launch")


class ForwardBench:
    def __init__(self, wl, dev, gated=False):
        import numpy as np
        import torch

        import synth
        self.wl = wl
        self.gated = gated
        x = synth.make_forward_inputs(wl)
        self.host = x
        self.r = self.r_host = None
        if gated:
            self.r_host, r_bits = synth.make_receptance(wl)
        if wl.dtype == "bf16":
            self.k = torch.from_numpy(x.k_bits.view(np.int16)).to(dev).view(torch.bfloat16)
            self.v = torch.from_numpy(x.v_bits.view(np.int16)).to(dev).view(torch.bfloat16)
            if gated:
                self.r = torch.from_numpy(r_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            self.k = torch.from_numpy(x.k).to(dev)
            self.v = torch.from_numpy(x.v).to(dev)
            if gated:
                self.r = torch.from_numpy(self.r_host).to(dev)
        self.w = torch.from_numpy(x.w).to(dev)
        self.u = torch.from_numpy(x.u).to(dev)
        self.y = torch.empty_like(self.k)
        es = 2 if wl.dtype == "bf16" else 4
        self.units = wl.B * wl.T * wl.C                       # tokens * channels per step
        # k, v (and r) read; y written; w, u
        self.alg_bytes = (4 if gated else 3) * es * self.units + 8 * wl.C
        self.dtype = "f32"                                    # arithmetic type
        self.io = "bf16" if wl.dtype == "bf16" else "f32"
        import linear_attention_rnn_forward_amd as wkv
        self.wkv = wkv

    def step(self):
        self.wkv.forward(self.k, self.v, self.w, self.u, out=self.y, r=self.r)

    def check_replay(self):
        """The graph's last output matches an eager launch's: bit for bit, or
        within the parity tolerance on the chunked path, whose look-back groups
        its combines by timing."""
        import torch
        y = self.y.clone().float()
        self.step()
        torch.cuda.synchronize()
        ref = self.y.float()
        scale = torch.clamp(ref.abs(), min=float(ref.square().mean().sqrt()))
        err = float(((y - ref).abs() / scale).max())
        if err > (2e-2 if self.io == "bf16" else 1e-4):
            raise RuntimeError(f"graph replay output differs from the eager launch ({err:.3e})")

    def config(self):
        name = self.wl.name + (", receptance gate fused (o = sigmoid(r) * wkv)" if self.gated else "")
        code = self.wkv.BF16 if self.io == "bf16" else self.wkv.F32
        return {"workload": name, "B": self.wl.B, "T": self.wl.T, "C": self.wl.C,
                "io_dtype": self.io, "state_dtype": "f32",
                "path": self.wkv.auto_path(self.wl.B, self.wl.T, self.wl.C, code)}

    def cpu_baseline(self, min_seconds=10.0):
        """The oracle over the whole workload, repeated until about
        min_seconds of wall time have passed; its last output is kept for the
        run's parity figure."""
        import oracle
        x = self.host
        passes = 0
        t0 = time.perf_counter()
        while True:
            if self.gated:
                self.y_oracle, _ = oracle.forward_gated(x.k, x.v, self.r_host, x.w, x.u)
            else:
                self.y_oracle, _ = oracle.forward(x.k, x.v, x.w, x.u)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
        return {"value": passes * self.units / dt, "unit": "tokens·channels/s",
                "cores": oracle.threads(), "kind": "oracle",
                "sample": f"the full workload ({self.units} tokens*channels), {passes} passes, "
                          f"{dt:.1f} s including fp64 conversion"}

    def parity(self):
        """Max guarded relative error of the timed run's output against the
        oracle's over the whole workload (guard: RMS of v), if the oracle ran."""
        y_ref = getattr(self, "y_oracle", None)
        if y_ref is None:
            return None
        from oracle.compare import guarded_rel_err, rms
        err = guarded_rel_err(self.y.float().cpu().numpy(), y_ref, rms(self.host.v))
        return {"max_guarded_rel_err": float(f"{err:.3e}"),
                "bar": 2e-2 if self.io == "bf16" else 1e-4,
                "against": "fp64 oracle, whole workload"}


class BackwardBench:
    """wkv_backward over the forward workload's shape: k, v and the output
    gradient gy read, gk, gv written (plus gw, gu [C]).  saved: the training
    pair's backward, wkv_backward_saved, from the states wkv_forward_save kept
    (made once before the timed region, as a training step's forward would)."""

    def __init__(self, wl, dev, saved=False):
        import numpy as np
        import torch

        import synth
        self.wl = wl
        x = synth.make_forward_inputs(wl)
        g, g_bits = synth.make_output_grad(wl)
        self.host = (x, g)
        if wl.dtype == "bf16":
            def put(bits):
                return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
            self.k, self.v, self.g = put(x.k_bits), put(x.v_bits), put(g_bits)
        else:
            self.k, self.v, self.g = (torch.from_numpy(a).to(dev) for a in (x.k, x.v, g))
        self.w = torch.from_numpy(x.w).to(dev)
        self.u = torch.from_numpy(x.u).to(dev)
        self.out = (torch.empty_like(self.k), torch.empty_like(self.k),
                    torch.empty(wl.C, device=dev), torch.empty(wl.C, device=dev))
        import linear_attention_rnn_forward_amd as wkv
        self.wkv = wkv
        self.saved = saved
        self.states = None
        self.save_cost = None
        if saved:
            self.ws = torch.empty(wkv.backward_saved_workspace_size(wl.B, wl.C), dtype=torch.uint8,
                                  device=dev)
            self.states = wkv.forward_save(self.k, self.v, self.w, self.u)[1]
            self.save_cost = self._save_cost(dev)
        else:
            self.ws = torch.empty(wkv.backward_workspace_size(wl.B, wl.T, wl.C), dtype=torch.uint8,
                                  device=dev)
        es = 2 if wl.dtype == "bf16" else 4
        self.units = wl.B * wl.T * wl.C
        # k, v, gy read and gk, gv written once; w, u read, gw, gu written
        # (the saved states, 1 byte per token-channel, are not counted)
        self.alg_bytes = 5 * es * self.units + 16 * wl.C
        # the kernel (forward-in-time phase, skipped when saved, then the
        # reverse phase) and the batch reduction
        self.launches = 2
        self.dtype = "f32"
        self.io = "bf16" if wl.dtype == "bf16" else "f32"

    def _save_cost(self, dev, n=20):
        """What saving the states adds to the forward: wkv_forward_save
        against the chained wkv_forward it runs, per launch, in us."""
        import torch
        y = torch.empty_like(self.k)
        st = torch.empty_like(self.states)
        stream = torch.cuda.current_stream(dev)

        def timed(fn):
            for _ in range(3):
                fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / n
        plain = timed(lambda: self.wkv.forward(self.k, self.v, self.w, self.u, out=y, path="chained"))
        save = timed(lambda: self.wkv.forward_save(self.k, self.v, self.w, self.u, out=y, states=st))
        return {"forward_chained_us": round(plain, 1), "forward_save_us": round(save, 1),
                "states_bytes": st.numel() * 4}

    def step(self):
        self.wkv.backward(self.k, self.v, self.w, self.u, self.g, out=self.out, workspace=self.ws,
                          states=self.states)

    def check_replay(self):
        """The graph's last outputs equal an eager launch's bit for bit (the
        backward has no timing-dependent order)."""
        import torch
        saved = [t.clone() for t in self.out]
        self.step()
        torch.cuda.synchronize()
        for a, b in zip(saved, self.out):
            if not torch.equal(a, b):
                raise RuntimeError("graph replay gradients differ from the eager launch")

    def config(self):
        c = {"workload": ("wkv_backward_saved (gradients of k, v, w, u from wkv_forward_save's "
                          "states) over " if self.saved else
                          "wkv_backward (gradients of k, v, w, u) over ") + self.wl.name,
             "B": self.wl.B, "T": self.wl.T, "C": self.wl.C, "io_dtype": self.io,
             "state_dtype": "f32"}
        if self.saved:
            c["saved_states"] = self.save_cost
        return c

    def cpu_baseline(self):
        import oracle
        x, g = self.host
        c0 = 1234 % self.wl.C
        sl = (slice(None), slice(None), slice(c0, c0 + 1))
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):      # the NumPy oracle on one core, as reported
            t0 = time.perf_counter()
            oracle.backward(x.k[sl], x.v[sl], x.w[c0:c0 + 1], x.u[c0:c0 + 1], g[sl])
            dt = time.perf_counter() - t0
        n = self.wl.B * self.wl.T
        return {"value": n / dt, "unit": "tokens·channels/s", "cores": 1, "kind": "oracle",
                "sample": f"channel {c0} of every batch row ({n} tokens*channels; the oracle is "
                          f"O(T^2) per column), {dt:.2f} s"}


class DecodeBench:
    """One wkv_step over [L,S,C] per step; k, v of 16 distinct tokens resident
    in HBM and used in turn; the state starts from a 512-token prefill."""

    def __init__(self, dev, ntok=16):
        import torch

        import linear_attention_rnn_forward_amd as wkv
        import synth
        import synth.device as sd
        wl = synth.DECODE
        self.wl = wl
        self.wkv = wkv
        w, u = synth.decode_params(wl)
        self.w = torch.from_numpy(w).to(dev)
        self.u = torch.from_numpy(u).to(dev)
        Ln, S, C = wl.L, wl.S, wl.C
        self.st = tuple(torch.empty((Ln, S, C), device=dev) for _ in range(3))
        kp = torch.empty((S, wl.prefill_T, C), device=dev)
        vp = torch.empty_like(kp)
        for l in range(Ln):
            sd.decode_prefill_kv(wl, l, kp, vp)
            wkv.forward(kp, vp, self.w[l], self.u[l], state_out=(self.st[0][l], self.st[1][l], self.st[2][l]))
        del kp, vp
        self.kb = torch.empty((ntok, Ln, S, C), device=dev)
        self.vb = torch.empty_like(self.kb)
        sd.decode_step_kv(wl, 0, ntok, self.kb, self.vb)
        self.y = torch.empty((Ln, S, C), device=dev)
        self.i = 0
        self.ntok = ntok
        self.units = Ln * S * C
        self.alg_bytes = 36 * self.units + 8 * Ln * C
        self.dtype = "f32"

    def step(self):
        j = self.i % self.ntok
        self.wkv.step(self.st, self.kb[j], self.vb[j], self.w, self.u, out=self.y, inplace=True)
        self.i += 1

    def begin_capture(self):
        self.i_capture = self.i

    def snapshot(self):
        self.st_before = tuple(s.clone() for s in self.st)

    def check_replay(self):
        """The replayed steps, re-run eagerly from the saved state, give the
        same state and output, bit for bit."""
        import torch
        st = self.st_before
        steps = self.i - self.i_capture
        for n in range(steps):
            j = (self.i_capture + n) % self.ntok
            y, st = self.wkv.step(st, self.kb[j], self.vb[j], self.w, self.u, inplace=True)
        torch.cuda.synchronize()
        if not (torch.equal(y, self.y) and all(torch.equal(a, b) for a, b in zip(st, self.st))):
            raise RuntimeError("graph replay of the decode steps differs from eager launches")
        self.st_before = None

    def config(self):
        return {"workload": self.wl.name, "L": self.wl.L, "S": self.wl.S, "C": self.wl.C,
                "io_dtype": "f32", "state_dtype": "f32"}

    def cpu_baseline(self):
        import numpy as np

        import oracle
        wl = self.wl
        rng = np.random.default_rng(0)
        Ls = 4   # a sample of 4 layers of the [32,256,4096] step, 10 steps
        a = np.zeros((Ls, wl.S, wl.C))
        b = np.ones((Ls, wl.S, wl.C))
        p = rng.normal(0, 1, (Ls, wl.S, wl.C))
        k = rng.normal(0, 1, (Ls, wl.S, wl.C))
        v = rng.normal(0, 1, (Ls, wl.S, wl.C))
        w = self.w[:Ls].cpu().numpy()
        u = self.u[:Ls].cpu().numpy()
        t0 = time.perf_counter()
        st = (a, b, p)
        for _ in range(10):
            _, st = oracle.step(st, k, v, w, u)
        dt = time.perf_counter() - t0
        units = 10 * Ls * wl.S * wl.C
        return {"value": units / dt, "unit": "tokens·channels/s", "cores": oracle.threads(),
                "kind": "oracle", "sample": f"10 steps over 4 of the 32 layers ({units} states)"}


class MatBench:
    """wkv_mat_forward (matrix-valued state, RWKV-5/6) over a [B,T,C] batch:
    r, k, v (and z per token) read, y written; no state in or out."""

    def __init__(self, wl, dev):
        import numpy as np
        import torch

        import linear_attention_rnn_forward_amd as wkv
        import synth
        self.wl = wl
        self.wkv = wkv
        x = synth.make_mat_inputs(wl)
        self.host = x
        if wl.dtype == "bf16":
            dv = lambda n: torch.from_numpy(x.bits[n].view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            dv = lambda n: torch.from_numpy(getattr(x, n)).to(dev)
        self.r, self.k, self.v = dv("r"), dv("k"), dv("v")
        self.z = dv("z") if wl.per_token_z else torch.from_numpy(x.z).to(dev)
        self.y = torch.empty_like(self.k)
        es = 2 if wl.dtype == "bf16" else 4
        self.units = wl.B * wl.T * wl.C
        self.alg_bytes = (5 if wl.per_token_z else 4) * es * self.units + \
            (0 if wl.per_token_z else 4 * wl.C)
        self.dtype = "f32"         # fp32 accumulation of bf16 matrix-core products

    def step(self):
        self.wkv.mat_forward(self.r, self.k, self.v, self.z, out=self.y)

    def check_replay(self):
        import torch
        y = self.y.clone()
        self.step()
        torch.cuda.synchronize()
        if not torch.equal(y, self.y):
            raise RuntimeError("graph replay of wkv_mat_forward differs from the eager launch")

    def config(self):
        return {"workload": self.wl.name, "B": self.wl.B, "T": self.wl.T, "H": self.wl.H,
                "C": self.wl.C, "head_dim": 64, "io_dtype": self.wl.dtype, "state_dtype": "f32"}

    def cpu_baseline(self):
        from threadpoolctl import threadpool_limits

        from oracle import matrix_state as ms
        x = self.host
        Ts = 512   # the first 512 tokens of every batch row and head
        z = x.z[:, :Ts] if self.wl.per_token_z else x.z
        with threadpool_limits(1):
            t0 = time.perf_counter()
            ms.forward(x.r[:, :Ts], x.k[:, :Ts], x.v[:, :Ts], z)
            dt = time.perf_counter() - t0
        n = self.wl.B * Ts * self.wl.C
        return {"value": n / dt, "unit": "tokens·channels/s", "cores": 1, "kind": "oracle",
                "sample": f"the first {Ts} tokens of every batch row and head ({n} tokens*channels), "
                          f"{dt:.2f} s"}


class MatDecodeBench:
    """One wkv_mat_step over [L,S] rows of H heads per step; r, k, v, z of
    `pool` distinct tokens resident in HBM and used in turn; the state starts
    at zero and the warm-up steps fill it."""

    def __init__(self, dev):
        import torch

        import linear_attention_rnn_forward_amd as wkv
        import synth
        wl = synth.MAT_DECODE
        self.wl = wl
        self.wkv = wkv
        x = synth.make_mat_decode_pool(wl)
        self.pool = {n: torch.from_numpy(getattr(x, n)).to(dev) for n in ("r", "k", "v", "z")}
        self.st = torch.zeros((wl.L, wl.S, wl.H, 64, 64), device=dev)
        self.y = torch.empty((wl.L, wl.S, wl.C), device=dev)
        self.i = 0
        self.units = wl.L * wl.S * wl.C
        # the state read and written (8 B per element), r, k, v, z read and y written
        self.alg_bytes = 8 * wl.L * wl.S * wl.H * 64 * 64 + 5 * 4 * self.units
        self.dtype = "f32"

    def step(self):
        j = self.i % self.wl.pool
        p = self.pool
        self.wkv.mat_step(self.st, p["r"][j], p["k"][j], p["v"][j], p["z"][j], out=self.y,
                          inplace=True)
        self.i += 1

    def begin_capture(self):
        self.i_capture = self.i

    def snapshot(self):
        self.st_before = self.st.clone()

    def check_replay(self):
        """The replayed steps, re-run eagerly from the saved state, give the
        same state and output, bit for bit."""
        import torch
        st = self.st_before
        p = self.pool
        for n in range(self.i - self.i_capture):
            j = (self.i_capture + n) % self.wl.pool
            y, st = self.wkv.mat_step(st, p["r"][j], p["k"][j], p["v"][j], p["z"][j], inplace=True)
        torch.cuda.synchronize()
        if not (torch.equal(y, self.y) and torch.equal(st, self.st)):
            raise RuntimeError("graph replay of the matrix-state decode differs from eager launches")
        self.st_before = None

    def config(self):
        wl = self.wl
        return {"workload": wl.name, "L": wl.L, "S": wl.S, "H": wl.H, "C": wl.C, "head_dim": 64,
                "io_dtype": "f32", "state_dtype": "f32"}

    def cpu_baseline(self):
        import numpy as np
        from threadpoolctl import threadpool_limits

        from oracle import matrix_state as ms
        wl = self.wl
        rows = 8   # 8 of the 2048 (layer, sequence) rows, every head, 4 steps
        p = {n: self.pool[n][:, 0, :rows].cpu().numpy() for n in self.pool}
        st = np.zeros((rows, wl.H, 64, 64))
        with threadpool_limits(1):
            t0 = time.perf_counter()
            for j in range(wl.pool):
                _, st = ms.step(st, p["r"][j], p["k"][j], p["v"][j], p["z"][j])
            dt = time.perf_counter() - t0
        n = wl.pool * rows * wl.C
        return {"value": n / dt, "unit": "tokens·channels/s", "cores": 1, "kind": "oracle",
                "sample": f"{wl.pool} steps of {rows} of the {wl.L * wl.S} rows ({n} tokens*channels), "
                          f"{dt:.2f} s"}


class CopyBench:
    """A plain device copy of 2 x 256 MiB (torch's copy kernel): known bytes, used
    to scale the HBM counters (FETCH_SIZE, WRITE_SIZE) of the WKV kernels."""

    def __init__(self, dev):
        import torch
        self.x = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        self.y = torch.empty_like(self.x)
        self.units = self.x.numel()
        self.alg_bytes = 2 * 4 * self.units
        self.dtype = "f32"

    def step(self):
        self.y.copy_(self.x)

    def check_replay(self):
        import torch
        if not torch.equal(self.x, self.y):
            raise RuntimeError("graph replay of the copy is wrong")

    def config(self):
        return {"workload": "device copy of 256 MiB (counter calibration)", "bytes": self.alg_bytes}

    def cpu_baseline(self):
        return None


class TokenShiftBench:
    def __init__(self, dev):
        import torch

        import linear_attention_rnn_forward_amd as wkv
        self.wkv = wkv
        B, T, C = 16, 4096, 2048
        g = torch.Generator(device="cpu").manual_seed(6)
        self.x = torch.randn((B, T, C), generator=g).to(torch.bfloat16).to(dev)
        self.mu = [torch.rand(C, generator=g).to(dev) for _ in range(3)]
        self.out = tuple(torch.empty_like(self.x) for _ in range(3))
        self.units = B * T * C
        self.alg_bytes = 4 * 2 * self.units + 12 * C
        self.dtype = "f32"
        self.shape = (B, T, C)

    def step(self):
        self.wkv.token_shift(self.x, *self.mu, out=self.out)

    def check_replay(self):
        import torch
        got = [t.clone() for t in self.out]
        ref = self.wkv.token_shift(self.x, *self.mu)   # fresh outputs
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(got, ref)):
            raise RuntimeError("graph replay of the token shift differs from the eager launch")

    def config(self):
        B, T, C = self.shape
        return {"workload": "token shift B=16 T=4096 C=2048 bf16", "B": B, "T": T, "C": C,
                "io_dtype": "bf16"}

    def cpu_baseline(self):
        import numpy as np

        import oracle
        x = self.x[:2].float().cpu().numpy()
        mus = [m.cpu().numpy() for m in self.mu]
        t0 = time.perf_counter()
        oracle.token_shift(x, *mus)
        dt = time.perf_counter() - t0
        return {"value": x.size / dt, "unit": "tokens·channels/s", "cores": oracle.threads(),
                "kind": "oracle", "sample": "2 of the 16 batch rows"}


def step_spread(bench, stream, n):
    """min / median / max duration of n eager steps, HIP events recorded on
    the launch stream between consecutive steps (launched back to back)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        bench.step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n))
    return {"min": round(d[0], 2), "median": round(d[n // 2], 2), "max": round(d[-1], 2), "n": n,
            "from": "eager steps right after the timed replay, HIP events between steps"}


def copy_ceiling(nbytes, dev, stream, n=20):
    """GB/s of a plain device copy moving nbytes in all (nbytes / 2 read,
    nbytes / 2 written): the rate this device gives a simple stream."""
    import torch
    half = max(int(nbytes // 2) // 4, 1)
    x = torch.ones(half, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(n):
        y.copy_(x)
    ev1.record(stream)
    torch.cuda.synchronize()
    t = ev0.elapsed_time(ev1) / 1e3 / n
    return 2 * 4 * half / t / 1e9


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bf16_main",
                    choices=["tiny", "small_lm", "bf16_main", "bf16_main_gated", "bf16_main_backward",
                             "bf16_main_backward_saved",
                             "long_ctx", "decode", "token_shift", "hbm_copy", "mat_main",
                             "mat_eagle", "mat_decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch each step from Python instead of replaying a HIP graph of the steps")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU kernel only: run it with --gpus 1 "
              "(the operator shards across GPUs without communication for batch x channels; "
              "that path is not built here).", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in synth.FORWARD_WORKLOADS:
        bench = ForwardBench(synth.FORWARD_WORKLOADS[args.workload], dev)
    elif args.workload == "bf16_main_gated":
        bench = ForwardBench(synth.BF16_MAIN, dev, gated=True)
    elif args.workload == "bf16_main_backward":
        bench = BackwardBench(synth.BF16_MAIN, dev)
    elif args.workload == "bf16_main_backward_saved":
        bench = BackwardBench(synth.BF16_MAIN, dev, saved=True)
    elif args.workload == "decode":
        bench = DecodeBench(dev)
    elif args.workload == "mat_main":
        bench = MatBench(synth.MAT_MAIN, dev)
    elif args.workload == "mat_eagle":
        bench = MatBench(synth.MAT_EAGLE, dev)
    elif args.workload == "mat_decode":
        bench = MatDecodeBench(dev)
    elif args.workload == "hbm_copy":
        bench = CopyBench(dev)
    else:
        bench = TokenShiftBench(dev)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        bench.step()
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        # the K steps as one HIP graph: the same kernels, launched without the
        # per-step Python and launch-queue gaps
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            bench.step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        getattr(bench, "begin_capture", lambda: None)()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                bench.step()
        torch.cuda.synchronize()
        graph.replay()   # untimed first replay
        torch.cuda.synchronize()
        getattr(bench, "snapshot", lambda: None)()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            bench.step()
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if graph is not None:
        bench.check_replay()
    # average duration of one launch on the launch stream: HIP events around the
    # timed region, divided by the launch count
    avg_kernel_s = ev0.elapsed_time(ev1) / 1e3 / args.steps

    spread = step_spread(bench, stream, args.steps)
    value = bench.units * args.steps / elapsed
    achieved = bench.alg_bytes / avg_kernel_s / 1e9
    copy_gbs = copy_ceiling(bench.alg_bytes, dev, stream)
    traffic = measured_traffic(args.workload)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic,
                "alg_bytes_per_launch": bench.alg_bytes,
                "launches_per_step": getattr(bench, "launches", 1),
                "avg_launch_us": round(avg_kernel_s * 1e6, 2)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = bench.cpu_baseline()
        if cpu is not None:
            cpu["value"] = float(f"{cpu['value']:.4g}")
    parity = getattr(bench, "parity", lambda: None)()
    line = {"metric": METRIC, "value": float(f"{value:.6g}"), "unit": "tokens·channels/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": bench.dtype, "data": "synthetic",
            "config": dict(bench.config(), launch="hip graph of the timed steps" if graph is not None
                           else "one launch per step"),
            "roofline": roofline, "cpu_baseline": cpu,
            "step_us": spread,
            "copy_ceiling": {"GB/s": round(copy_gbs, 1), "frac": round(achieved / copy_gbs, 4),
                             "bytes": bench.alg_bytes, "kernel": "torch device copy, same bytes"},
            "parity": parity}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
