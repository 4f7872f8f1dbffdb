#!/usr/bin/env python3
"""Benchmark of the k-quant decode hot path on one MI355X.

A step is one decode token through the 52-layer FFN weight stream: per layer a
Q4_K gate matvec (19968 x 6656), a Q4_K up matvec with the SiLU-gated epilogue,
a Q6_K down matvec (6656 x 19968) and the fused dual-eps tail; the activation
is chained layer to layer (the weight arena of Ch 19 "The down projection +
residual", section 19.6, times 52 layers).  Weights are seeded synthetic
(13.44 GB of distinct bytes, larger than the 256 MB Infinity Cache), resident
in HBM before timing.  The pass is captured once as a HIP graph and replayed.

Printed: one JSON line (rank 0) with the headline metric -- achieved HBM GB/s
of the pass -- plus the roofline of the dominant kernel (timed with HIP events
on the launch stream), per-kernel numbers, the measured read-stream ceiling,
isolated matvec rates with weight rotation, and the CPU oracle's rate on a
bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import struct
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HIDDEN, FFN, LAYERS = 6656, 19968, 52
QDIM, KVDIM, VOCAB = 4096, 256, 202048  # attention projection and vocabulary sizes
PEAK_HBM_GBPS = 8000.0
Q4K_BLOCK, Q6K_BLOCK = 144, 210
FULL_MODEL_TOKEN_BYTES = 16_756_681_056  # pages' per-token weight bytes (Ch 1, section 1.3)


def q4k_bytes(n, k):
    return n * (k // 256) * Q4K_BLOCK


def q6k_bytes(n, k):
    return n * (k // 256) * Q6K_BLOCK


# Algorithmic bytes per launch: every weight byte once, activations in and out.
BYTES = {
    "gate": q4k_bytes(FFN, HIDDEN) + 4 * HIDDEN + 4 * FFN,
    "up_silu": q4k_bytes(FFN, HIDDEN) + 4 * HIDDEN + 4 * FFN + 4 * FFN,
    "down": q6k_bytes(HIDDEN, FFN) + 4 * FFN + 4 * HIDDEN,
    # tail: read projected, read+write residual, write next_in, read two gains
    "tail": 4 * HIDDEN * 6,
}
# gate and up in one launch: both matrices, x in, mid out
GATE_UP_BYTES = 2 * q4k_bytes(FFN, HIDDEN) + 4 * HIDDEN + 4 * FFN


def staged_bytes(group, k):
    """Algorithmic bytes of a staged activation: 3 byte limbs per input, a scale
    and a sum per group (the 16 bytes of padding per 128 inputs in the stored
    form are layout, not counted)."""
    return 3 * k + 8 * (k // group)


# the staged pass: activations cross launches in the consumer's staged form
# (groups of 32 inputs for Q4_K, 16 for Q6_K); mid is also written as f32
STAGED_BYTES = {
    "gate_up_staged": 2 * q4k_bytes(FFN, HIDDEN) + staged_bytes(32, HIDDEN) + 4 * FFN
                      + staged_bytes(16, FFN),
    "down_staged": q6k_bytes(HIDDEN, FFN) + staged_bytes(16, FFN) + 4 * HIDDEN,
    "tail_staged": 4 * HIDDEN * 6 + staged_bytes(32, HIDDEN),
    # the previous layer's tail fused into gate+up: the tail's four inputs and
    # the residual it writes, both matrices, mid f32 and staged
    "tail_gate_up": 2 * q4k_bytes(FFN, HIDDEN) + 5 * 4 * HIDDEN + 4 * FFN + staged_bytes(16, FFN),
}
# one token through the pass: per layer gate+up (x in, mid out), down, tail; plus the entry norm.
# The same count serves every schedule of the pass, so their rates compare work for work.
PASS_BYTES = LAYERS * (GATE_UP_BYTES + BYTES["down"] + BYTES["tail"]) + BYTES["tail"]
WEIGHT_BYTES_PASS = LAYERS * (2 * q4k_bytes(FFN, HIDDEN) + q6k_bytes(HIDDEN, FFN))
KERNEL_SYMBOL = {
    "gate": "q45k_matvec_kernel<4, ..., false>",
    "up_silu": "q45k_matvec_kernel<4, ..., true>",
    "down": "q6k_matvec_kernel",
    "tail": "tail_reg_kernel",
    "gate_up": "q4k_gate_up_kernel",
    "gate_up_staged": "q4k_gate_up_kernel (staged x in, staged mid out)",
    "down_staged": "q6k_matvec_kernel (staged x in)",
    "tail_staged": "tail_reg_kernel (staged next_in out)",
    "tail_gate_up": "q4k_gate_up_kernel<..., true> (previous tail fused in, staged mid out)",
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


LIB_PATH = os.path.join(ROOT, "quant_weight_matvec_amd", "libkq.so")
# the timed instantiations (mangled-name prefixes) whose machine code a
# committed counter summary covers: q4k_gate_up_kernel<8, 3, 1, 16, true> and
# q6k_matvec_kernel<8, 3, 1, 8>.  Only these are hashed, since the compiler
# may schedule other instantiations of the same template differently when
# unrelated code in the file changes.
PMC_KERNELS = {"gate_up": "q4k_gate_up_kernelILi8ELi3ELi1ELi16ELb1E",
               "down": "q6k_matvec_kernelILi8ELi3ELi1ELi8EE"}


def _elf_sections(elf: bytes):
    """Section headers of a little-endian ELF64 image: name, type, addr, offset, size, link."""
    shoff = struct.unpack_from("<Q", elf, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    secs = []
    for i in range(shnum):
        name, typ, _fl, addr, off, size, link = struct.unpack_from("<IIQQQQI", elf, shoff + i * shentsize)
        secs.append({"name_off": name, "type": typ, "addr": addr, "off": off, "size": size, "link": link})
    names = secs[shstrndx]["off"]
    for sec in secs:
        start = names + sec["name_off"]
        sec["name"] = elf[start:elf.index(b"\0", start)].decode()
    return secs


def kernel_code(name_part: str, lib_path: str = LIB_PATH, objects: bool = False):
    """[(symbol, machine code bytes)] of every gfx950 kernel whose symbol
    contains `name_part`, sorted by symbol, read from the code objects the
    library embeds (uncompressed clang offload bundles in its .hip_fatbin
    section); [] if the library or the section is missing.  With `objects`
    the data objects instead (the kernel descriptors)."""
    if not os.path.exists(lib_path):
        return []
    with open(lib_path, "rb") as f:
        data = f.read()
    fat = [s for s in _elf_sections(data) if s["name"] == ".hip_fatbin"]
    if not fat:
        return []
    fat = data[fat[0]["off"]:fat[0]["off"] + fat[0]["size"]]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    found = []
    pos = fat.find(magic)
    while pos >= 0:
        p = pos + len(magic)
        n_entries = struct.unpack_from("<Q", fat, p)[0]
        p += 8
        for _ in range(n_entries):
            off, size, tlen = struct.unpack_from("<QQQ", fat, p)
            triple = fat[p + 24:p + 24 + tlen].decode()
            p += 24 + tlen
            if not triple.endswith("gfx950"):
                continue
            co = fat[pos + off:pos + off + size]
            secs = _elf_sections(co)
            for symtab in (s for s in secs if s["type"] == 2):  # SHT_SYMTAB
                strs = secs[symtab["link"]]["off"]
                for i in range(symtab["size"] // 24):
                    st_name, st_info, _o, shndx, value, sz = struct.unpack_from(
                        "<IBBHQQ", co, symtab["off"] + 24 * i)
                    nm = co[strs + st_name:co.index(b"\0", strs + st_name)].decode()
                    kind = 1 if objects else 2  # STT_OBJECT (descriptors) or STT_FUNC
                    if (st_info & 0xF) == kind and sz and name_part in nm:
                        sec = secs[shndx]
                        start = sec["off"] + value - sec["addr"]
                        found.append((nm, co[start:start + sz]))
        pos = fat.find(magic, pos + len(magic))
    return sorted(found)


def kernel_descriptors(name_part: str, lib_path: str = LIB_PATH):
    """{symbol: (LDS bytes, private bytes per lane)} of every gfx950 kernel
    whose symbol contains `name_part`, from its kernel descriptor (the 64-byte
    `<symbol>.kd` object of the code object: group_segment_fixed_size at
    offset 0, private_segment_fixed_size at offset 4).  Private bytes are
    register spills or per-lane arrays kept in memory."""
    out = {}
    for nm, body in kernel_code(name_part, lib_path, objects=True):
        if nm.endswith(".kd") and len(body) >= 8:
            out[nm[:-3]] = struct.unpack_from("<II", body, 0)
    return out


def kernel_code_hash(name_part: str, lib_path: str = LIB_PATH):
    """Hash of the machine code of every kernel `kernel_code` finds. A
    committed counter summary is used only while this matches: edits that
    leave the kernel's code unchanged keep it valid, any change to that code
    drops it. None if no such kernel is found."""
    code = kernel_code(name_part, lib_path)
    if not code:
        return None
    h = hashlib.sha256()
    for nm, body in code:
        h.update(nm.encode())
        h.update(body)
    return h.hexdigest()[:16]


class FFNChain:
    """Device buffers of the 52-layer chain and the launches of one pass."""

    def __init__(self, torch, kq, I, layers=LAYERS):
        self.torch, self.kq = torch, kq
        dev = torch.device("cuda")
        self.layers = layers
        t0 = time.time()
        self.Wg, self.Wu, self.Wd, self.gp, self.gn = [], [], [], [], []
        for l in range(layers):
            self.Wg.append(torch.from_numpy(I.q4k_matrix(FFN, HIDDEN, stream=I.stream_id(4, l, I.ROLE_W_GATE))).to(dev))
            self.Wu.append(torch.from_numpy(I.q4k_matrix(FFN, HIDDEN, stream=I.stream_id(4, l, I.ROLE_W_UP))).to(dev))
            self.Wd.append(torch.from_numpy(I.q6k_matrix(HIDDEN, FFN, stream=I.stream_id(4, l, I.ROLE_W_DOWN))).to(dev))
            self.gp.append(torch.from_numpy(I.gains_f32(HIDDEN, stream=I.stream_id(4, l, I.ROLE_GPOST))).to(dev))
            self.gn.append(torch.from_numpy(I.gains_f32(HIDDEN, stream=I.stream_id(4, l, I.ROLE_GNEXT))).to(dev))
        torch.cuda.synchronize()
        log(f"generated and uploaded {layers} layers ({WEIGHT_BYTES_PASS * layers / LAYERS / 1e9:.2f} GB) "
            f"in {time.time() - t0:.1f}s")
        self.res0 = torch.from_numpy(I.normal_f32(HIDDEN, stream=I.stream_id(4, 0, I.ROLE_RESID))).to(dev)
        self.residual = self.res0.clone()
        self.x = [torch.empty(HIDDEN, device=dev), torch.empty(HIDDEN, device=dev)]
        self.g = torch.empty(FFN, device=dev)
        self.mid = torch.empty(FFN, device=dev)
        self.p = torch.empty(HIDDEN, device=dev)
        self.zeros = torch.zeros(HIDDEN, device=dev)
        self.ones = torch.ones(HIDDEN, device=dev)
        u8 = torch.uint8
        self.xst = [torch.empty(kq.kq_staged_bytes(kq.KQ_QTYPE_Q4K, HIDDEN), dtype=u8, device=dev)
                    for _ in range(2)]
        self.mid_s = torch.empty(kq.kq_staged_bytes(kq.KQ_QTYPE_Q6K, FFN), dtype=u8, device=dev)
        self.R = [self.residual, torch.empty(HIDDEN, device=dev)]  # residual ping-pong
        self.table = kq.kq_ffn_layer_table([(self.Wg[l], self.Wu[l], self.Wd[l], self.gp[l],
                                             self.gn[l]) for l in range(layers)])
        self.pass_ws = torch.empty(kq.kq_ffn_pass_workspace_bytes(HIDDEN, FFN), dtype=torch.uint8,
                                   device=dev)

    def entry_norm(self):
        # x_0 = rms_norm(residual, 1e-5) with unit gain: the tail with a zero
        # projection leaves the residual unchanged and emits exactly that.
        self.kq.kq_fused_residual_norm(self.residual, self.zeros, self.x[0], self.ones, self.ones,
                                       1, HIDDEN, 1e-8, 1e-5)

    def entry_norm_staged(self):
        self.kq.kq_fused_residual_norm_staged(self.residual, self.zeros, self.x[0], self.xst[0],
                                              self.kq.KQ_QTYPE_Q4K, self.ones, self.ones, 1,
                                              HIDDEN, 1e-8, 1e-5)

    def calls_staged(self, l):
        """The layer as three launches with staged activations: gate+up+SiLU
        reads x staged and writes mid staged, down reads it, the tail writes
        the next x staged."""
        kq = self.kq
        xs, xn, xsn = self.xst[l % 2], self.x[(l + 1) % 2], self.xst[(l + 1) % 2]
        Q4, Q6 = kq.KQ_QTYPE_Q4K, kq.KQ_QTYPE_Q6K
        return (
            ("gate_up_staged", lambda: kq.kq_ffn_gate_up_q4k_staged(
                self.Wg[l], self.Wu[l], xs, self.mid, self.mid_s, Q6, FFN, HIDDEN)),
            ("down_staged", lambda: kq.kq_matvec_staged(Q6, self.Wd[l], self.mid_s, self.p,
                                                        HIDDEN, FFN)),
            ("tail_staged", lambda: kq.kq_fused_residual_norm_staged(
                self.residual, self.p, xn, xsn, Q4, self.gp[l], self.gn[l], 1, HIDDEN, 1e-8, 1e-5)),
        )

    def calls_fusedtail(self, l):
        """The layer as two launches: the previous layer's tail fused into
        this layer's gate+up+SiLU (layer 0: the entry norm, i.e. the tail with
        a zero projection and unit gains), then the down matvec on staged mid.
        The residual alternates between two buffers: every workgroup of the
        fused launch reads the old one while one of them writes the new one."""
        kq = self.kq
        Q6 = kq.KQ_QTYPE_Q6K
        pp, gp, gn = (self.zeros, self.ones, self.ones) if l == 0 else \
            (self.p, self.gp[l - 1], self.gn[l - 1])
        R = self.R
        return (
            ("tail_gate_up", lambda: kq.kq_ffn_tail_gate_up_q4k(
                R[l % 2], pp, gp, gn, R[(l + 1) % 2], None, self.Wg[l], self.Wu[l], self.mid,
                self.mid_s, Q6, FFN, HIDDEN, 1e-8, 1e-5)),
            ("down_staged", lambda: kq.kq_matvec_staged(Q6, self.Wd[l], self.mid_s, self.p,
                                                        HIDDEN, FFN)),
        )

    def lib_pass(self):
        """The whole pass as one library call: kq_ffn_pass_q4k_q6k enqueues the
        launches of calls_fusedtail for every layer, then the last tail."""
        self.kq.kq_ffn_pass_q4k_q6k(self.table, self.R[0], self.x[0], None, self.pass_ws,
                                    self.pass_ws.numel(), HIDDEN, FFN, 1e-8, 1e-5)

    def final_tail(self):
        """The last layer's tail (after the fused pass): residual and x_out."""
        L = self.layers
        self.kq.kq_fused_residual_norm(self.R[L % 2], self.p, self.x[0], self.gp[L - 1],
                                       self.gn[L - 1], 1, HIDDEN, 1e-8, 1e-5)

    def calls(self, l):
        kq = self.kq
        x, xn = self.x[l % 2], self.x[(l + 1) % 2]
        return (
            ("gate", lambda: kq.kq_matvec_q4k(self.Wg[l], x, self.g, FFN, HIDDEN)),
            ("up_silu", lambda: kq.kq_matvec_q4k(self.Wu[l], x, self.mid, FFN, HIDDEN, self.g)),
            ("down", lambda: kq.kq_matvec_q6k(self.Wd[l], self.mid, self.p, HIDDEN, FFN)),
            ("tail", lambda: kq.kq_fused_residual_norm(self.residual, self.p, xn, self.gp[l],
                                                       self.gn[l], 1, HIDDEN, 1e-8, 1e-5)),
        )

    def calls_fused(self, l):
        """The layer as three launches: gate+up+SiLU, down, tail."""
        kq = self.kq
        x, xn = self.x[l % 2], self.x[(l + 1) % 2]
        return (
            ("gate_up", lambda: kq.kq_ffn_gate_up_q4k(self.Wg[l], self.Wu[l], x, self.mid, FFN, HIDDEN)),
            ("down", lambda: kq.kq_matvec_q6k(self.Wd[l], self.mid, self.p, HIDDEN, FFN)),
            ("tail", lambda: kq.kq_fused_residual_norm(self.residual, self.p, xn, self.gp[l],
                                                       self.gn[l], 1, HIDDEN, 1e-8, 1e-5)),
        )

    def run_pass(self, mode="4launch"):
        """One token: the entry norm, then every layer as 4 launches ("4launch"),
        3 with gate and up fused ("fused"), 3 with staged activations
        ("staged"); or every layer as 2 launches with each tail fused into the
        next gate+up, then the last tail ("fusedtail")."""
        if mode == "fusedtail":
            for l in range(self.layers):
                for _, fn in self.calls_fusedtail(l):
                    fn()
            self.final_tail()
            return
        if mode == "staged":
            self.entry_norm_staged()
        else:
            self.entry_norm()
        calls = {"4launch": self.calls, "fused": self.calls_fused, "staged": self.calls_staged}[mode]
        for l in range(self.layers):
            for _, fn in calls(l):
                fn()

    def per_kernel_us(self, reps):
        """Average duration of each per-op kernel: one graph per kernel holding
        its launch for every layer (distinct weights, so no cache reuse),
        replayed reps times; time / (reps * layers)."""
        torch = self.torch
        out = {}
        four = ("gate", "up_silu", "down", "tail")
        st = ("gate_up_staged", "down_staged", "tail_staged")
        for name in four + ("gate_up",) + st + ("tail_gate_up",):
            if name == "tail_gate_up":
                pick = lambda l: self.calls_fusedtail(l)[0][1]
            elif name == "gate_up":
                pick = lambda l: self.calls_fused(l)[0][1]
            elif name in st:
                pick = lambda l, i=st.index(name): self.calls_staged(l)[i][1]
            else:
                pick = lambda l, i=four.index(name): self.calls(l)[i][1]
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for l in range(self.layers):
                    pick(l)()
            torch.cuda.synchronize()
            for _ in range(3):  # steady clocks before timing
                g.replay()
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ea.record()
            for _ in range(reps):
                g.replay()
            eb.record()
            torch.cuda.synchronize()
            out[name] = ea.elapsed_time(eb) * 1e3 / (reps * self.layers)
            del g
        return out


class EventLog:
    def __init__(self, torch):
        self.torch = torch
        self.items = []

    def pair(self):
        E = self.torch.cuda.Event
        return E(enable_timing=True), E(enable_timing=True)

    def note(self, name, a, b):
        self.items.append((name, a, b))

    def summary(self):
        self.torch.cuda.synchronize()
        out = {}
        for name, a, b in self.items:
            out.setdefault(name, []).append(a.elapsed_time(b) * 1e3)  # us
        return {k: np.array(v) for k, v in out.items()}


def graph_of(torch, calls):
    """The launches of `calls` (a list of no-argument functions) captured as
    one graph on a side stream."""
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s_):
        for c in calls:
            c()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, launches, reps=5, warm=2):
    """Per-launch microseconds of each of `reps` replays of a graph of
    `launches` back-to-back launches (HIP events on the replay stream), after
    `warm` untimed replays: (median, CV, all)."""
    for _ in range(warm):
        g.replay()
    times = []
    for _ in range(reps):
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ea.record()
        g.replay()
        eb.record()
        torch.cuda.synchronize()
        times.append(ea.elapsed_time(eb) * 1e3 / launches)
    t = np.array(times)
    return float(np.median(t)), float(np.std(t) / np.mean(t)), [round(float(v), 3) for v in t]


# the matvec weight streams the probe windows are matched to
WINDOWS = {"q4k_19968x6656": q4k_bytes(FFN, HIDDEN), "q6k_6656x19968": q6k_bytes(HIDDEN, FFN),
           "gate_up_pair": 2 * q4k_bytes(FFN, HIDDEN)}


def read_ceiling(torch, kq, nbytes=4 << 30, reps=5, launches=52, layers=LAYERS):
    """The HBM read ceiling the matvecs are compared with.
    (1) One pass over a 4 GiB buffer for a sweep of probe variants (workgroup
    size and count, loads in flight per thread, non-temporal or normal loads,
    grid-stride or one contiguous chunk per workgroup); median of `reps`.
    (2) With the best variant and with the chunked one, windows of the sizes
    the matvecs stream, at rotating offsets through the 4 GiB buffer, as a
    graph of `launches` back-to-back launches timed like the isolated matvecs
    (so the two compare like with like).
    (3) The pass's own shape with no arithmetic: per layer one window of the
    gate+up pair's bytes, then one of the down's, for `layers` layers (2 per
    layer launches back to back in one graph), at offsets advancing through
    the 4 GiB buffer, so no window is still in the Infinity Cache when read;
    and the same bytes as one window per layer (what merging a layer's two
    launches could reach at best)."""
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(7)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 64 * 16, dtype=torch.int32, device="cuda")
    E = torch.cuda.Event
    sweep = []
    for block in (256, 512, 1024):
        for per_cu in (1, 2, 4, 8, 16):
            grid = cus * per_cu
            if grid * block > cus * 2048 * 4:  # beyond four workgroups' worth of waves per CU
                continue
            for unroll in (4, 8, 16):
                for flags in (0, 1, 2, 3):
                    kq.kq_probe_read_bw(buf, nbytes, out, grid, block, unroll, flags)
                    ts = []
                    for _ in range(reps):
                        a, b = E(enable_timing=True), E(enable_timing=True)
                        a.record()
                        kq.kq_probe_read_bw(buf, nbytes, out, grid, block, unroll, flags)
                        b.record()
                        torch.cuda.synchronize()
                        ts.append(a.elapsed_time(b) / 1e3)
                    sweep.append({"grid": grid, "block": block, "unroll": unroll,
                                  "nontemporal": bool(flags & 1), "chunked": bool(flags & 2),
                                  "GBps": round(nbytes / float(np.median(ts)) / 1e9, 1)})
    sweep.sort(key=lambda r: -r["GBps"])
    best = sweep[0]
    best_chunk = next(r for r in sweep if r["chunked"])
    windows = {}
    for name, wb in WINDOWS.items():
        wb16 = (wb + 4095) // 4096 * 4096
        nwin = nbytes // wb16
        for label, v in (("best", best), ("chunked", best_chunk)):
            fl = (1 if v["nontemporal"] else 0) | (2 if v["chunked"] else 0)
            calls = [lambda o=(i % nwin) * wb16, v=v, fl=fl: kq.kq_probe_read_bw(
                buf[o // 4:], wb16, out, v["grid"], v["block"], v["unroll"], fl)
                for i in range(launches)]
            g = graph_of(torch, calls)
            med, cv, _ = time_graph(torch, g, launches, reps)
            del g
            windows[f"{name}_{label}"] = {"bytes": wb16, "windows_rotated": int(nwin),
                                          "us_median": round(med, 3), "us_cv": round(cv, 4),
                                          "GBps": round(wb16 / med / 1e3, 1)}
    pass_shaped = {}
    per_layer = {"": [WINDOWS["gate_up_pair"], WINDOWS["q6k_6656x19968"]],
                 "_one_launch_per_layer": [WINDOWS["gate_up_pair"] + WINDOWS["q6k_6656x19968"]]}
    for (suffix, win), (label, v) in itertools.product(per_layer.items(),
                                                       (("best", best), ("chunked", best_chunk))):
        seq = win * layers
        label = label + suffix
        fl = (1 if v["nontemporal"] else 0) | (2 if v["chunked"] else 0)
        calls, off, total = [], 0, 0
        for wb in seq:
            wb16 = (wb + 4095) // 4096 * 4096
            if off + wb16 > nbytes:
                off = 0
            calls.append(lambda o=off, n=wb16, v=v, fl=fl: kq.kq_probe_read_bw(
                buf[o // 4:], n, out, v["grid"], v["block"], v["unroll"], fl))
            off += wb16
            total += wb16
        g = graph_of(torch, calls)
        med, cv, _ = time_graph(torch, g, 1, reps)
        del g
        pass_shaped[label] = {"layers": layers, "launches": len(calls), "bytes": total,
                              "ms_median": round(med / 1e3, 4), "cv": round(cv, 4),
                              "GBps": round(total / med / 1e3, 1)}
    del buf, out
    torch.cuda.empty_cache()
    return {"GBps_4GiB_best": best["GBps"], "best_variant": best, "best_chunked": best_chunk,
            "sweep_top": sweep[:8], "sweep_worst": sweep[-3:], "size_matched": windows,
            "pass_shaped": pass_shaped}


def isolated_matvecs(torch, kq, I, reps=5, launches=52):
    """Single matvecs at the FFN shapes, timed as the pass runs them: a graph
    of `launches` back-to-back launches, each on the next of >= 1 GiB of
    weight copies (so the Infinity Cache cannot serve them), replayed `reps`
    times between HIP events on the replay stream; per-launch time = replay
    time / launches; median and CV over the replays.  Each shape with x in
    f32 (every workgroup encodes it) and with x staged beforehand (the form
    the pass hands between launches)."""
    out = {}
    cases = [("q4k_19968x6656", "q4k", FFN, HIDDEN), ("q4k_6656x19968", "q4k", HIDDEN, FFN),
             ("q6k_6656x19968", "q6k", HIDDEN, FFN), ("q5k_19968x6656", "q5k", FFN, HIDDEN)]
    QTYPES = {"q4k": kq.KQ_QTYPE_Q4K, "q5k": kq.KQ_QTYPE_Q5K, "q6k": kq.KQ_QTYPE_Q6K}
    FNS = {"q4k": kq.kq_matvec_q4k, "q5k": kq.kq_matvec_q5k, "q6k": kq.kq_matvec_q6k}
    for name, qt, n, k in cases:
        qtype = QTYPES[qt]
        W = torch.from_numpy(I.weight_matrix(qt, n, k, stream=777)).cuda()
        ncopy = max(2, int(np.ceil((1 << 30) / W.numel())))
        copies = [W] + [W.clone() for _ in range(ncopy - 1)]
        x = torch.from_numpy(I.normal_f32(k, stream=778)).cuda()
        xs = torch.empty(kq.kq_staged_bytes(qtype, k), dtype=torch.uint8, device="cuda")
        kq.kq_stage_activation(qtype, x, xs, k)
        y = torch.empty(n, device="cuda")
        fn = FNS[qt]
        nl = max(launches, ncopy)
        for form, call, xbytes in (
                ("", lambda c: fn(c, x, y, n, k), 4 * k),
                ("_staged", lambda c: kq.kq_matvec_staged(qtype, c, xs, y, n, k), xs.numel())):
            g = graph_of(torch, [lambda c=copies[i % ncopy]: call(c) for i in range(nl)])
            med, cv, all_ = time_graph(torch, g, nl, reps)
            del g
            nbytes = W.numel() + xbytes + 4 * n
            out[name + form] = {"us_median": round(med, 3), "us_cv": round(cv, 4),
                                "us_replays": all_, "launches_per_replay": nl,
                                "GBps": round(nbytes / med / 1e3, 1),
                                "frac_peak": round(nbytes / med / 1e3 / PEAK_HBM_GBPS, 4),
                                "copies_rotated": ncopy, "bytes": nbytes}
            if not form:  # the automatic shape of the f32 form (the staged form may differ)
                out[name]["shape"] = list(kq.kq_tune_get_shape(qtype, n, k))
        del copies, W
        torch.cuda.empty_cache()
    return out


# The decode matvec shapes outside the FFN (Ch 10 "The forward pass at a
# glance", section 10.3): the attention projections as one group on one input
# (Q, K, V, gate), K or V alone, o_proj, and the LM head, in both weight types.
DECODE_SHAPES = [
    ("qkvg_group", [QDIM, KVDIM, KVDIM, QDIM], HIDDEN),
    ("kv_alone", [KVDIM], HIDDEN),
    ("q_alone", [QDIM], HIDDEN),
    ("o_proj", [HIDDEN], QDIM),
    ("lm_head", [VOCAB], HIDDEN),
]


def decode_shapes(torch, kq, I, reps=5, launches=52, max_launches=1200):
    """Each shape as a graph of back-to-back launches, each launch on the next
    of >= 1 GiB of weight copies (at most max_launches copies; fewer copies
    of a small matrix still exceed the 256 MB Infinity Cache), median and CV
    over `reps` replays.  Bytes per launch: the weights once, x in, y out."""
    out = {}
    for qt in ("q4k", "q6k"):
        qtype = kq.KQ_QTYPE_Q4K if qt == "q4k" else kq.KQ_QTYPE_Q6K
        rowb = lambda k: (k // 256) * (Q4K_BLOCK if qt == "q4k" else Q6K_BLOCK)
        for name, rows, k in DECODE_SHAPES:
            wb = [n * rowb(k) for n in rows]
            set_bytes = sum(wb)
            ncopy = int(min(max_launches, max(2, np.ceil((1 << 30) / set_bytes))))
            host = [I.weight_matrix(qt, n, k, stream=800 + i) for i, n in enumerate(rows)]
            buf = torch.empty(ncopy * set_bytes, dtype=torch.uint8, device="cuda")
            first = torch.from_numpy(np.concatenate([h.reshape(-1) for h in host])).cuda()
            for c in range(ncopy):
                buf[c * set_bytes:(c + 1) * set_bytes].copy_(first)
            del host, first
            offs = np.concatenate([[0], np.cumsum(wb)[:-1]])
            x = torch.from_numpy(I.normal_f32(k, stream=810)).cuda()
            ys = [torch.empty(n, device="cuda") for n in rows]
            base = buf.data_ptr()

            def call(c):
                Ws = [base + c * set_bytes + int(o) for o in offs]
                if len(rows) == 1:
                    fn = kq.kq_matvec_q4k if qt == "q4k" else kq.kq_matvec_q6k
                    fn(Ws[0], x, ys[0], rows[0], k)
                else:
                    kq.kq_matvec_group(qtype, Ws, ys, rows, x, k)
            nl = max(launches, ncopy)
            g = graph_of(torch, [lambda c=(i % ncopy): call(c) for i in range(nl)])
            med, cv, _ = time_graph(torch, g, nl, reps)
            del g, buf
            torch.cuda.empty_cache()
            nbytes = set_bytes + 4 * k + 4 * sum(rows)
            out[f"{name}_{qt}"] = {"rows": rows, "k": k, "bytes": nbytes, "copies_rotated": ncopy,
                                   "launches_per_replay": nl, "us_median": round(med, 3),
                                   "us_cv": round(cv, 4), "GBps": round(nbytes / med / 1e3, 1),
                                   "frac_peak": round(nbytes / med / 1e3 / PEAK_HBM_GBPS, 4),
                                   "shape": list(kq.kq_tune_get_shape(qtype, sum(rows), k))}
            log(f"  {name}_{qt}: {med:.2f} us, {nbytes / med / 1e3:.0f} GB/s")
    return out


def verify_pass(torch, kq, chain, ms=(1, 2, 3, 4, 8, 16), reps=3):
    """The speculative-verify batch through the 52-layer FFN pass (Ch 10
    "The forward pass at a glance", sections 10.2-10.3; Ch 36 section 36.4):
    for M activation rows, per layer kq_ffn_gate_up_q4k_small_m (gate, up and
    the SiLU product), kq_matmul_small_m (Q6_K down) and kq_fused_residual_norm
    over the M rows; the entry norm first.  At M = 1 the tail goes into the
    gate+up launch instead, as in the decode pass: kq_ffn_tail_gate_up_q4k runs
    layer l-1's tail (layer 0: the entry norm, a zero projection with unit
    gains) in front of layer l's gate+up, and one kq_fused_residual_norm ends
    the pass.  Captured as one graph and replayed; tokens/s = M / time per
    pass, GB/s = the pass's weight bytes / time."""
    Q4, Q6 = kq.KQ_QTYPE_Q4K, kq.KQ_QTYPE_Q6K
    L = chain.layers
    out = {}
    res0 = torch.randn(16, HIDDEN, device="cuda")
    ones, zeros = torch.ones(HIDDEN, device="cuda"), torch.zeros(16, HIDDEN, device="cuda")
    for m in ms:
        need = max(kq.kq_matmul_small_m_workspace_bytes(Q4, FFN, HIDDEN, m),
                   kq.kq_matmul_small_m_workspace_bytes(Q6, HIDDEN, FFN, m))
        ws = torch.zeros(max(need, 256) // 4, dtype=torch.int32, device="cuda")
        R = res0[:m].clone()
        X = [torch.empty(m, HIDDEN, device="cuda") for _ in range(2)]
        mid = torch.empty(m, FFN, device="cuda")
        P = torch.empty(m, HIDDEN, device="cuda")

        fused = m == 1
        R2 = [R, torch.empty_like(R)]

        def run():
            kq.kq_fused_residual_norm(R, zeros[:m], X[0], ones, ones, m, HIDDEN)
            for l in range(L):
                kq.kq_ffn_gate_up_q4k_small_m(chain.Wg[l], chain.Wu[l], X[l % 2], HIDDEN, mid, FFN,
                                              FFN, HIDDEN, m, ws, need)
                kq.kq_matmul_small_m(Q6, chain.Wd[l], mid, FFN, P, HIDDEN, HIDDEN, FFN, m, ws, need)
                kq.kq_fused_residual_norm(R, P, X[(l + 1) % 2], chain.gp[l], chain.gn[l], m, HIDDEN)

        def run_fused():
            for l in range(L):
                first = l == 0
                kq.kq_ffn_tail_gate_up_q4k(
                    R2[l % 2], zeros[0] if first else P, ones if first else chain.gp[l - 1],
                    ones if first else chain.gn[l - 1], R2[(l + 1) % 2], None, chain.Wg[l],
                    chain.Wu[l], mid, None, 0, FFN, HIDDEN)
                kq.kq_matmul_small_m(Q6, chain.Wd[l], mid, FFN, P, HIDDEN, HIDDEN, FFN, m, ws, need)
            kq.kq_fused_residual_norm(R2[L % 2], P, X[1], chain.gp[L - 1], chain.gn[L - 1], m,
                                      HIDDEN)
        body = run_fused if fused else run
        body()
        torch.cuda.synchronize()
        g = graph_of(torch, [body])
        # M = 1: the tail in front of the one-launch gate+up; M = 2 and 3:
        # gate+up in one dot-path launch (default), then down and the tail;
        # above: two gate+up launches.  Running the M tails inside the
        # dot-path launch measured slower at M = 2 and 3 (4.51 and 5.16 ms
        # against 4.12-4.23 and 4.61-4.75), so those keep the separate tail.
        launches = 1 + L * (2 if fused else (3 if m <= 3 else 4))
        # more warm replays than the default: the first replays of a 3 ms
        # graph after its capture read up to 4 % slow
        med, cv, _ = time_graph(torch, g, 1, reps, warm=4)
        del g
        wb = WEIGHT_BYTES_PASS * L // LAYERS
        out[f"m{m}"] = {"us_per_pass": round(med, 1), "us_cv": round(cv, 4),
                        "tokens_per_s": round(m / med * 1e6, 1),
                        "weight_GBps": round(wb / med / 1e3, 1), "launches": launches}
        log(f"  verify pass M={m}: {med / 1e3:.3f} ms, {m / med * 1e6:.0f} tokens/s")
    return out


def embedding_lookup(torch, kq, I, reps=5, launches=52):
    """kq_embedding of 16 tokens (a verify batch) from the [202048 x 6656]
    Q4_K and Q5_K tables: 16 rows of 3744 / 4576 B gathered and dequantized."""
    out = {}
    for qt, qtype in (("q4k", kq.KQ_QTYPE_Q4K), ("q5k", kq.KQ_QTYPE_Q5K)):
        E = torch.from_numpy(I.weight_matrix(qt, VOCAB, HIDDEN, stream=820)).cuda()
        tok = torch.from_numpy(I.token_ids(16 * launches, VOCAB, stream=821)).cuda()
        o = torch.empty(16, HIDDEN, device="cuda")
        g = graph_of(torch, [lambda i=i: kq.kq_embedding(qtype, E, VOCAB, HIDDEN, tok[16 * i:],
                                                         16, o) for i in range(launches)])
        med, cv, _ = time_graph(torch, g, launches, reps)
        del g, E
        torch.cuda.empty_cache()
        out[qt] = {"tokens": 16, "us_median": round(med, 3), "us_cv": round(cv, 4)}
    return out


def small_m_sweep(torch, kq, I, ms=(1, 2, 3, 4, 8, 16), reps=5, launches=52):
    """kq_matmul_small_m at the verify shapes, M = 1..16: per-launch time from a
    graph of 52 launches over >= 1 GiB of rotated weight copies (so the
    Infinity Cache cannot serve them), median and CV of 5 replays, with GB/s
    (weights once + X + Y) and GFLOP/s."""
    out = {}
    cases = [("q4k_19968x6656", kq.KQ_QTYPE_Q4K, "q4k", FFN, HIDDEN),
             ("q6k_6656x19968", kq.KQ_QTYPE_Q6K, "q6k", HIDDEN, FFN)]
    for name, qti, qt, n, k in cases:
        W = torch.from_numpy(I.weight_matrix(qt, n, k, stream=779)).cuda()
        ncopy = max(2, int(np.ceil((1 << 30) / W.numel())))
        copies = [W] + [W.clone() for _ in range(ncopy - 1)]
        X = torch.from_numpy(I.normal_f32((16, k), stream=780)).cuda()
        Y = torch.empty((16, n), device="cuda")
        res = {}
        for m in ms:
            nbytes = kq.kq_matmul_small_m_workspace_bytes(qti, n, k, m)
            ws = torch.zeros(max(nbytes, 256) // 4, dtype=torch.int32, device="cuda")
            call = lambda c: kq.kq_matmul_small_m(qti, c, X, k, Y, n, n, k, m, ws, nbytes)
            for c in copies:
                call(c)
            # graph of 52 launches over the rotated copies (a copy may repeat,
            # far enough apart that the Infinity Cache no longer holds it)
            g = graph_of(torch, [lambda c=copies[i % ncopy]: call(c) for i in range(launches)])
            us, cv, all_us = time_graph(torch, g, launches, reps=reps, warm=3)
            b = W.numel() + 4 * m * (n + k)
            res[f"m{m}"] = {"us": round(us, 3), "us_cv": round(cv, 4), "us_replays": all_us,
                            "GBps": round(b / us / 1e3, 1),
                            "frac_peak": round(b / us / 1e3 / PEAK_HBM_GBPS, 4),
                            "GFLOPs": round(2.0 * m * n * k / us / 1e3, 1), "bytes": b}
            del g, ws
        out[name] = {"copies_rotated": ncopy, **res}
        del copies, W
        torch.cuda.empty_cache()
    return out


def small_m_cases(torch, kq, I, launches=8):
    """Each small-M kernel choice at the verify shapes, `launches` eager
    launches per case over rotated weight copies, cases in a fixed order (for
    a counter run, whose per-dispatch rows follow this order): the M = 1
    matvec, the dot path and the matrix-core kernel at the same M (each
    forced where it is not the default), and the verify gate+up."""
    Q4, Q6 = kq.KQ_QTYPE_Q4K, kq.KQ_QTYPE_Q6K
    mats = {"q4k": (Q4, FFN, HIDDEN), "q6k": (Q6, HIDDEN, FFN)}
    cases = [("q4k", 1, None), ("q4k", 2, 4), ("q4k", 2, 0), ("q4k", 4, 4), ("q4k", 4, 0),
             ("q4k", 16, 0), ("q6k", 1, None), ("q6k", 2, 4), ("q6k", 2, 0), ("q6k", 16, 0),
             ("gate_up", 1, None), ("gate_up", 2, 3), ("gate_up", 2, 0), ("gate_up", 3, 3),
             ("gate_up", 3, 0)]
    W = {}
    for qt, (qti, n, k) in mats.items():
        w = torch.from_numpy(I.weight_matrix(qt, n, k, stream=781)).cuda()
        W[qt] = [w] + [w.clone() for _ in range(max(2, int(np.ceil((1 << 30) / w.numel()))) - 1)]
    X = torch.from_numpy(I.normal_f32((16, FFN), stream=782)).cuda()
    Y = torch.empty((16, FFN), device="cuda")
    order = []
    for name, m, rows in cases:
        qt = "q4k" if name == "gate_up" else name
        qti, n, k = mats[qt]
        if name == "gate_up":  # the two-launch form on the matrix cores
            kq.kq_tune_set_gate_up_rows(-1 if rows is None else rows)
            kq.kq_tune_set_small_m_rows(qti, 0)
        else:
            kq.kq_tune_set_small_m_rows(qti, -1 if rows is None else rows)
        nb = kq.kq_matmul_small_m_workspace_bytes(qti, n, k, m)
        ws = torch.zeros(max(nb, 256) // 4, dtype=torch.int32, device="cuda")
        cp = W[qt]
        for i in range(launches):
            if name == "gate_up":
                kq.kq_ffn_gate_up_q4k_small_m(cp[i % len(cp)], cp[(i + 1) % len(cp)], X, k, Y, n, n,
                                              k, m, ws, nb)
            else:
                kq.kq_matmul_small_m(qti, cp[i % len(cp)], X, k, Y, n, n, k, m, ws, nb)
        torch.cuda.synchronize()
        if m == 1:
            path, per = ("one launch" if name == "gate_up" else "matvec"), 1
        elif rows:
            path, per = ("dot path, one launch" if name == "gate_up" else "dot path"), 1
        elif name == "gate_up":
            path, per = "matrix cores, two launches", 2
        else:
            path, per = "matrix cores", 1
        order.append({"case": f"{name} M={m} {path}", "dispatches": launches * per})
        del ws
    kq.kq_tune_set_small_m_rows(Q4, -1)
    kq.kq_tune_set_small_m_rows(Q6, -1)
    kq.kq_tune_set_gate_up_rows(-1)
    return order


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(I, budget_s=8.0):
    """The oracle (plain C, binary64) on a bounded sample of the same pass:
    layer 0's FFN (gate, up, silu, down, tail) at full size, repeated for
    about budget_s seconds, on one thread and on all the cores this process
    may use (at most 16: the CPU share of one GPU on the box)."""
    import oracle
    o = oracle.get()
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(16, avail))
    Wg = I.q4k_matrix(FFN, HIDDEN, stream=I.stream_id(4, 0, I.ROLE_W_GATE))
    Wu = I.q4k_matrix(FFN, HIDDEN, stream=I.stream_id(4, 0, I.ROLE_W_UP))
    Wd = I.q6k_matrix(HIDDEN, FFN, stream=I.stream_id(4, 0, I.ROLE_W_DOWN))
    gp, gn = I.gains_f32(HIDDEN, stream=I.stream_id(4, 0, I.ROLE_GPOST)), I.gains_f32(HIDDEN, stream=I.stream_id(4, 0, I.ROLE_GNEXT))
    res = I.normal_f32(HIDDEN, stream=I.stream_id(4, 0, I.ROLE_RESID)).astype(np.float64)
    x = o.rms_norm(res, 1e-5)
    layer_bytes = WEIGHT_BYTES_PASS / LAYERS

    def run(nt):
        runs, t0 = 0, time.time()
        while True:
            o.ffn_layer(Wg, Wu, Wd, HIDDEN, FFN, x, res, gp, gn, nthreads=nt)
            runs += 1
            if time.time() - t0 >= budget_s:
                break
        dt = time.time() - t0
        return runs, dt, layer_bytes * runs / dt / 1e9

    r1, d1, v1 = run(1)
    rn, dn, vn = run(threads)
    return {"value": round(vn, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{rn} run(s) of layer 0 of the 52-layer FFN pass (gate, up, silu, down, "
                      f"tail; {layer_bytes / 1e6:.1f} MB of weights each) on {threads} threads in "
                      f"{dn:.1f}s; pass-equivalent {dn / rn * LAYERS:.1f} s/token",
            "cpu_model": cpu_model(), "cores_available": avail,
            "single_thread": {"value": round(v1, 3), "unit": "GB/s", "cores": 1,
                              "sample": f"{r1} run(s) of the same layer on one thread in {d1:.1f}s; "
                                        f"pass-equivalent {d1 / r1 * LAYERS:.1f} s/token"}}


def load_pmc(symbol_key: str, code_hash):
    """HBM traffic per launch from a committed counter summary, if it was
    taken on the kernel's current machine code; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{symbol_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if code_hash is None or d.get("kernel_code_hash") != code_hash:
        return None
    return d.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=LAYERS, help=argparse.SUPPRESS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip read ceiling and isolated matvecs")
    ap.add_argument("--eager", action="store_true", help="time uncaptured launches instead of a graph")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run one 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--only", choices=("pass", "isolated", "small_m", "small_m_cases", "probe",
                                       "cpu", "shapes", "embedding"),
                    help="run one section alone (for profiler runs) and print its results")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode path is "
              "built and measured on a single MI355X. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import quant_weight_matvec_amd as kq
    from quant_weight_matvec_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    kq.lib()
    log(kq.kq_build_info())
    code_hash = {k: kernel_code_hash(v) for k, v in PMC_KERNELS.items()}

    if args.calibration_copy:
        # a plain copy kernel of known size: 1 GiB read, 1 GiB written
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1073741824 bytes read and written")
        del src, dst
        torch.cuda.empty_cache()

    if args.only and args.only != "pass":
        log(f"section {args.only} only")
        sec = {"isolated": lambda: {"isolated_matvec": isolated_matvecs(torch, kq, I)},
               "small_m": lambda: {"small_m": small_m_sweep(torch, kq, I)},
               "small_m_cases": lambda: {"small_m_cases": small_m_cases(torch, kq, I)},
               "probe": lambda: {"read_ceiling": read_ceiling(torch, kq)},
               "shapes": lambda: {"decode_shapes": decode_shapes(torch, kq, I)},
               "embedding": lambda: {"embedding": embedding_lookup(torch, kq, I)},
               "cpu": lambda: {"cpu_baseline": cpu_baseline(I)}}[args.only]()
        print(json.dumps({"section": args.only, **sec, "build": kq.kq_build_info()}), flush=True)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return
    if args.only == "pass":
        args.no_extras = args.no_cpu_baseline = True

    chain = FFNChain(torch, kq, I, args.layers)
    layers = args.layers
    pass_bytes = layers * (GATE_UP_BYTES + BYTES["down"] + BYTES["tail"]) + BYTES["tail"]
    stream = torch.cuda.current_stream()

    def timed(fn, steps):
        torch.cuda.synchronize()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ea.record()
        for _ in range(steps):
            fn()
        eb.record()
        torch.cuda.synchronize()
        return ea.elapsed_time(eb) / steps, time.perf_counter() - t0

    def capture(fn):
        """fn's launches captured once as a graph (None with --eager)."""
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        if args.eager:
            return None
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        return g

    # ---- the step as timed: one graph replay of the whole pass: per layer the
    # previous tail (the entry norm for layer 0) fused with gate+up+SiLU, then
    # the down matvec on staged mid; then the last tail
    ft_pass = chain.lib_pass
    graph_t = capture(ft_pass)
    log(f"timing {args.steps} steps (graph of kq_ffn_pass_q4k_q6k: 2 launches per layer, "
        "tail fused into gate+up)")
    step_fn = (lambda: graph_t.replay()) if graph_t is not None else ft_pass
    ms_per_step, wall = timed(step_fn, args.steps)
    value = pass_bytes / (ms_per_step * 1e-3) / 1e9
    # the same K steps timed five more times, after the timed region: the
    # spread of the headline figure (value itself is the timed region's)
    repeats = [timed(step_fn, args.steps)[0] for _ in range(5)]
    rep_med = float(np.median(repeats))
    headline_spread = {"ms_per_step": [round(t, 4) for t in repeats],
                       "median_ms": round(rep_med, 4),
                       "cv": round(float(np.std(repeats) / np.mean(repeats)), 5),
                       "steps_each": args.steps}

    # ---- the same pass other ways, reported beside it
    staged_pass = lambda: chain.run_pass("staged")
    graph_s = capture(staged_pass)
    staged_ms, _ = timed((lambda: graph_s.replay()) if graph_s is not None else staged_pass,
                         args.steps)
    fused_pass = lambda: chain.run_pass("fused")
    graph_f = capture(fused_pass)
    fused_ms, _ = timed((lambda: graph_f.replay()) if graph_f is not None else fused_pass,
                        args.steps)
    four_pass = lambda: chain.run_pass("4launch")
    graph4 = capture(four_pass)
    per_op4_ms, _ = timed((lambda: graph4.replay()) if graph4 is not None else four_pass,
                          args.steps)
    per_kernel = chain.per_kernel_us(max(2, min(args.steps, 5))) if graph_t is not None else {}
    kernels = {}
    for name, avg in per_kernel.items():  # per-op kernels: graph of one launch per layer
        nb = GATE_UP_BYTES if name == "gate_up" else (STAGED_BYTES.get(name) or BYTES[name])
        gbps = nb / (avg * 1e-6) / 1e9
        kernels[name] = {"symbol": KERNEL_SYMBOL[name], "us_avg": round(avg, 3),
                         "bytes_per_launch": nb, "GBps": round(gbps, 1),
                         "frac_peak": round(gbps / PEAK_HBM_GBPS, 4),
                         "timing": f"graph of {layers} back-to-back launches (one per layer), "
                                   "HIP events on the replay stream"}
    # the dominant kernel of the timed step: gate+up+SiLU (150 MB of its ~260 MB per layer)
    dk = kernels.get("tail_gate_up")
    roofline = None
    if dk is not None:
        roofline = {"kernel": dk["symbol"], "bound": "hbm", "achieved": dk["GBps"],
                    "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": dk["frac_peak"],
                    "traffic": load_pmc("gate_up", code_hash["gate_up"]),
                    "bytes_per_launch": dk["bytes_per_launch"], "us_avg": dk["us_avg"]}
    alternatives = {
        "graph_3_launches_per_layer_staged_activations": {
            "ms_per_step": round(staged_ms, 4),
            "GBps": round(pass_bytes / (staged_ms * 1e-3) / 1e9, 1),
            "launches_per_step": 3 * layers + 1},
        "graph_3_launches_per_layer_f32_activations": {
            "ms_per_step": round(fused_ms, 4), "GBps": round(pass_bytes / (fused_ms * 1e-3) / 1e9, 1),
            "launches_per_step": 3 * layers + 1},
        "graph_4_launches_per_layer": {"ms_per_step": round(per_op4_ms, 4),
                                       "GBps": round(pass_bytes / (per_op4_ms * 1e-3) / 1e9, 1),
                                       "launches_per_step": 4 * layers + 1},
    }

    extras = {}
    if not args.no_extras:
        log("verify batch through the 52-layer pass")
        extras["verify_pass"] = verify_pass(torch, kq, chain)
        log("read-stream ceiling probe")
        rc = read_ceiling(torch, kq, layers=layers)
        extras["read_ceiling"] = rc
        extras["read_ceiling_GBps"] = rc["GBps_4GiB_best"]
        # the timed pass against the same stream read with no arithmetic
        ps = rc["pass_shaped"]
        ro = min(ps[k]["ms_median"] for k in ("best", "chunked"))
        ro1 = min(ps[k]["ms_median"] for k in ps if k.endswith("_one_launch_per_layer"))
        extras["pass_vs_read_only_pass"] = {"read_only_ms": ro, "pass_ms": round(ms_per_step, 4),
                                            "frac": round(ro / ms_per_step, 4),
                                            "read_only_one_launch_per_layer_ms": ro1}
        if roofline is not None:
            roofline["frac_of_read_ceiling"] = round(dk["GBps"] / rc["GBps_4GiB_best"], 4)
            roofline["frac_of_size_matched_read"] = round(
                dk["GBps"] / rc["size_matched"]["gate_up_pair_best"]["GBps"], 4)
        chain = graph_t = graph_s = graph_f = graph4 = None  # free 13.4 GB before the isolated runs
        torch.cuda.empty_cache()
        log("isolated matvecs with weight rotation")
        extras["isolated_matvec"] = isolated_matvecs(torch, kq, I)
        log("small-M verify matmul sweep")
        extras["small_m"] = small_m_sweep(torch, kq, I)
        log("other decode matvec shapes")
        extras["decode_shapes"] = decode_shapes(torch, kq, I)
        log("embedding lookup")
        extras["embedding"] = embedding_lookup(torch, kq, I)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(I)

    rec = {
        "metric": "achieved HBM GB/s (% of peak) for Q4_K/Q6_K matvec; equiv. decode tokens/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8 quants x i8 limbs -> i32, f32",
        "data": "synthetic (seeded Q4_K/Q6_K superblocks, N(0,1) activations, N(1,0.1) gains)",
        "config": {"workload": "ffn52: one decode token through 52 FFN layers (Q4_K gate+up 19968x6656, "
                               "SiLU product, Q6_K down 6656x19968, fused dual-eps tail)",
                   "hidden": HIDDEN, "ffn": FFN, "layers": args.layers, "tokens_per_step": 1,
                   "weight_bytes_per_step": WEIGHT_BYTES_PASS * args.layers // LAYERS,
                   "algorithmic_bytes_per_step": pass_bytes,
                   "timing": "one graph replay per step of kq_ffn_pass_q4k_q6k, which enqueues "
                             "per layer the previous layer's tail (or the entry norm) fused with "
                             "gate, up and SiLU (writing mid, and mid staged) and the Q6_K down matvec on "
                             "it, then the last dual-eps tail; 105 launches"},
        "alternatives": alternatives,
        "frac_peak": round(value / PEAK_HBM_GBPS, 4),
        "tokens_per_s": round(1e3 / ms_per_step, 2),
        "headline_repeats": headline_spread,
        "full_model_equiv_tokens_per_s": round(value * 1e9 / FULL_MODEL_TOKEN_BYTES, 2),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "kernel_code_hash": code_hash,
        "build": kq.kq_build_info(),
    }
    rec.update(extras)
    print(json.dumps(rec), flush=True)
    # Drop the graphs and device buffers and let the device drain before the
    # interpreter exits, so no captured graph or tensor outlives the runtime
    # (and a profiler's own teardown) at exit.
    chain = graph_t = graph_s = graph_f = graph4 = None  # noqa: F841
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
