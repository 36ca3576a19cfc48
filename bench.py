#!/usr/bin/env python3
"""Benchmark of the BitLinear forward on one MI355X.

One step = one pass of the whole hot path over one layer set of the workload:
  prefill leg (M = the workload's large token count):
    gamma + quantize-and-pack of every fp32 master weight   (grouped: 2 launches)
    int8 activation quantization of every input             (grouped: 1 launch)
    ternary x int8 product + rescale epilogue               (grouped: 1 launch)
  decode leg (M = 1, weights packed once outside timing):
    int8 activation quantization + streaming product + epilogue, fused  (grouped: 1 launch)
Inputs are seeded synthetic tensors (``workloads``) resident in HBM before timing starts.
Weights (fp32 masters for the prefill leg, packed words for the decode leg) and prefill
activations rotate through distinct copies totalling about 1 GB, so each step reads them
from HBM rather than from the 256 MB last-level cache.

Output: one JSON line.  ``value`` is the step's algorithmic int8 operations (2 M N K summed
over the prefill products) divided by the measured step time; decode GB/s, per-kernel
durations, roofline fractions and the CPU-oracle baseline are reported beside it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "BitLinear fwd: decode GB/s & prefill int8 TOPS, % of MI355X roofline"
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, published (no sparsity)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "bit_gemm_02_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--min-warmup-s", type=float, default=0.5,
                    help="keep running untimed warm-up steps until this much wall time has "
                         "passed (after at least --warmup steps): the clocks of a GPU that was "
                         "idle take tens of milliseconds of this load to settle")
    ap.add_argument("--workload", default="c5_qwen3_4b_layer",
                    choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--prefill-tokens", type=int, default=None,
                    help="override the prefill token count (default: the workload's largest)")
    ap.add_argument("--rotate-bytes", type=float, default=1e9,
                    help="bytes of distinct weight/activation copies to cycle through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="target seconds of oracle work for the CPU baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for counter scaling)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --copy-calibration run into profiles/traffic.json")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="turn rocprofv3 --pmc counter_collection.csv files (one per counter pass) "
                         "into a per-kernel table of MFMA utilisation, instruction mix, waits, LDS "
                         "bank conflicts and cache figures")
    ap.add_argument("--simds", type=int, default=1024,
                    help="SIMDs of the profiled GPU, for --summarize-counters (MI355X: 256 x 4)")
    ap.add_argument("--xcds", type=int, default=8,
                    help="XCDs of the profiled GPU (GRBM_GUI_ACTIVE is summed over them)")
    ap.add_argument("--layer", action="store_true",
                    help="time the whole layer chain (six launches per layer, residuals and the "
                         "FFN activation included) instead of the step; prints its own JSON line")
    ap.add_argument("--train", action="store_true",
                    help="time the training-side products (weight-only forward, input and weight "
                         "gradients through the STE, transposed packing) over the workload's "
                         "matrices at the prefill token count; prints its own JSON line")
    ap.add_argument("--verbose", action="store_true")
    return ap.parse_args()


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def source_hash(names: str) -> str:
    """Hash of the code a kernel is built from ("a.hip+b.hpp": every file, in order), with
    comments and whitespace runs taken out, so that counters stay attached to a kernel whose
    comments alone changed."""
    h = hashlib.sha256()
    for name in names.split("+"):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            code = _COMMENT.sub(" ", f.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def mixed_one_launch(wl: workloads.Workload, M_pre: int, M_dec: int = 1) -> bool:
    """Whether bitlinear_forward_mixed runs the step's products and decode leg as one launch:
    every product has more than 16 tokens on 128 x 128 tiles (fewer than 256 units of
    256 x 256 outputs; larger sets take 128 x 256 tiles), and the decode calls are fused
    with one activation dtype (always here)."""
    big = sum(-(-M_pre // 256) * -(-m.N // 256) for m in wl.matrices)
    return M_pre > 16 and big < 256 and M_dec <= 4


def decode_on_tiles(wl: workloads.Workload, M_pre: int) -> bool:
    """Whether the step's one-token decode leg runs on the decode tile layout (packed once,
    outside timing, from the two-bit rows): where the leg is a launch of its own (the products
    take 128 x 256 tiles) and every projection fits the one-token kernel."""
    return (not mixed_one_launch(wl, M_pre) and
            all(m.K % 64 == 0 and m.K <= 12288 for m in wl.matrices))


def prefill_on_quad_rows(wl: workloads.Workload, M_pre: int) -> bool:
    """Whether the step's prefill weights are quantized into (or packed once as) the quad-row
    layout and the products read them there: where the products are a launch of their own
    (128 x 256 tiles) and every matrix fits the layout (N % 4 == 0, K % 128 == 0)."""
    return (not mixed_one_launch(wl, M_pre) and M_pre > 16 and
            all(m.N % 4 == 0 and m.K % 128 == 0 for m in wl.matrices))


def gemv_layout(name: str) -> str:
    """'b3', 'tiles' or 'rows' for a gemv_kernel<S, BF16, PAIR, NORM, B3, TL> name."""
    args = name.split("(")[0].split("<", 1)[1].rstrip(">").split(",")
    args = [a.strip() for a in args]
    if args[4] == "true":
        return "b3"
    return "tiles" if len(args) > 5 and args[5] == "true" else "rows"


class Setup:
    """Device buffers and pre-built grouped problem tables for one workload."""

    def __init__(self, torch, bl, wl: workloads.Workload, M_pre: int, rotate_bytes: float):
        self.torch, self.bl, self.wl = torch, bl, wl
        dev = "cuda"
        mats = wl.matrices
        self.count = len(mats)
        self.M_pre = M_pre
        self.M_dec = 1
        t = torch

        # Host inputs (seeded).
        if wl.weights == "fp32":
            W_host = [workloads.weight_fp32(wl, i) for i in range(self.count)]
        else:
            W_host = None
        X_pre = [workloads.activations(wl, i, M_pre) for i in range(self.count)]
        X_dec = [workloads.activations(wl, i, self.M_dec) for i in range(self.count)]
        self.host = dict(W=W_host, X_pre=X_pre, X_dec=X_dec)

        def to_dev(a):
            if a.dtype == np.uint16:
                return t.from_numpy(a.view(np.int16)).to(dev).view(t.bfloat16)
            return t.from_numpy(np.ascontiguousarray(a)).to(dev)

        norms = [to_dev(workloads.norm_weight(wl, i)) if m.norm else None for i, m in enumerate(mats)]
        self.norms = norms

        # Rotating copies of the prefill-leg inputs (fp32 masters + activations).
        per_copy = sum(x.nbytes for x in X_pre) + (sum(w.nbytes for w in W_host) if W_host else 0)
        self.R_pre = int(max(1, min(64, np.ceil(rotate_bytes / per_copy))))
        base_X = [to_dev(x) for x in X_pre]
        self.X_pre = [[x.clone() for x in base_X] for _ in range(self.R_pre)]
        if W_host is not None:
            base_W = [to_dev(w) for w in W_host]
            self.W_pre = [[w.clone() for w in base_W] for _ in range(self.R_pre)]
        else:
            self.W_pre = None
        del base_X

        # Packed weights for the prefill product (written by the in-step quantization, or
        # packed once from pre-ternarized codes).
        self.P_pre = [t.empty((m.N, m.K // 16), dtype=t.int32, device=dev) for m in mats]
        self.g_pre = [t.empty(1, dtype=t.float32, device=dev) for m in mats]
        self.quad = prefill_on_quad_rows(wl, M_pre)
        if W_host is None:
            for i, m in enumerate(mats):
                bl.pack_codes(to_dev(workloads.weight_codes(wl, i)), self.P_pre[i])
                self.g_pre[i].fill_(wl.code_gamma)

        # Decode weights: packed once outside timing, replicated to distinct addresses.
        if W_host is not None:
            dec_packed = bl.quantize_weights_grouped([to_dev(w) for w in W_host])
        else:
            dec_packed = [(P.clone(), g) for P, g in zip(self.P_pre, self.g_pre)]
        if self.quad and W_host is None:
            # Pre-packed codes go to the quad-row layout once (the in-step quantization writes
            # that layout itself).
            self.P_pre = [bl.pack_quad_rows(P) for P in self.P_pre]
        packed_bytes = sum(p.numel() * 4 for p, _ in dec_packed)
        self.R_dec = int(max(1, min(4096, np.ceil(rotate_bytes / packed_bytes))))
        self.P_dec = [[p.clone() for p, _ in dec_packed] for _ in range(self.R_dec)]
        # The same decode weights in the base-3 layout (five codes per byte), for the
        # base-3 decode figure reported beside the step (not part of the step).
        self.B3_dec = [[bl.pack_b3(p) for p in Ps] for Ps in self.P_dec]
        # ... and in the decode tile layout, which the step's decode leg reads where it is a
        # launch of its own (the two-bit rows are then reported beside it).
        self.dec_tiles = decode_on_tiles(wl, M_pre)
        self.T_dec = [[bl.pack_tiles(p, m.K) for p, m in zip(Ps, mats)] for Ps in self.P_dec]
        self.g_dec = [g.clone() for _, g in dec_packed]
        self.X_dec = [to_dev(x) for x in X_dec]

        # Outputs.
        self.act_pre = [(t.empty((M_pre, m.K), dtype=t.int8, device=dev),
                         t.empty(M_pre, dtype=t.float32, device=dev)) for m in mats]
        self.act_dec = [(t.empty((1, m.K), dtype=t.int8, device=dev),
                         t.empty(1, dtype=t.float32, device=dev)) for m in mats]
        self.Y_pre = [t.empty((M_pre, m.N), dtype=t.float32, device=dev) for m in mats]
        self.Y_dec = [t.empty((1, m.N), dtype=t.float32, device=dev) for m in mats]
        # Weight-quantization workspace: large enough for the one-read form (each fp32 master
        # read once; the library takes it for sets of 64 MB and more).
        shapes = (bl._WeightProblem * self.count)()
        for i, m in enumerate(mats):
            shapes[i] = bl._WeightProblem(None, None, None, m.N, m.K)
        self.one_read_bytes = bl.quantize_weights_one_read_workspace_bytes(shapes, self.count)
        self.one_read = (W_host is not None and
                         sum(4 * m.N * m.K for m in mats) >= 64 << 20)
        self.ws = t.empty(max(16, bl.quantize_weights_workspace_bytes(self.count),
                              self.one_read_bytes if self.one_read else 0),
                          dtype=t.uint8, device=dev)
        self._build_tables()

    def _build_tables(self):
        """ctypes problem arrays, one per rotation copy, so the timed loop only calls C."""
        import ctypes
        bl = self.bl
        mats = self.wl.matrices
        n = self.count
        self.wq_tables = []
        if self.W_pre is not None:
            for r in range(self.R_pre):
                arr = (bl._WeightProblem * n)()
                for i, m in enumerate(mats):
                    arr[i] = bl._WeightProblem(self.W_pre[r][i].data_ptr(), self.P_pre[i].data_ptr(),
                                               self.g_pre[i].data_ptr(), m.N, m.K)
                self.wq_tables.append(arr)
        self.aq_pre_tables = []
        for r in range(self.R_pre):
            arr = (bl._ActProblem * n)()
            for i, m in enumerate(mats):
                X = self.X_pre[r][i]
                g = self.norms[i]
                dt = bl.BL_BF16 if X.dtype == self.torch.bfloat16 else bl.BL_F32
                arr[i] = bl._ActProblem(X.data_ptr(), None if g is None else g.data_ptr(),
                                        self.act_pre[i][0].data_ptr(), self.act_pre[i][1].data_ptr(),
                                        self.M_pre, m.K, dt, 1e-6)
            self.aq_pre_tables.append(arr)
        arr = (bl._ForwardProblem * n)()
        for i, m in enumerate(mats):
            arr[i] = bl._ForwardProblem(self.act_pre[i][0].data_ptr(), self.act_pre[i][1].data_ptr(),
                                        self.P_pre[i].data_ptr(), self.g_pre[i].data_ptr(),
                                        self.Y_pre[i].data_ptr(), None, self.M_pre, m.N, m.K)
        self.fwd_pre_table = arr
        ex = (bl._ForwardExProblem * n)()
        for i, m in enumerate(mats):
            ex[i] = bl._ForwardExProblem(self.act_pre[i][0].data_ptr(), self.act_pre[i][1].data_ptr(),
                                         self.P_pre[i].data_ptr(), self.g_pre[i].data_ptr(),
                                         self.Y_pre[i].data_ptr(), None, None, self.M_pre, m.N, m.K)
        self.fwd_pre_ex_table = ex
        # Decode leg: the fused layer call (activation quantization inside the product).
        self.lin_dec_tables = []
        for r in range(self.R_dec):
            arr = (bl._LinearProblem * n)()
            for i, m in enumerate(mats):
                X = self.X_dec[i]
                g = self.norms[i]
                dt = bl.BL_BF16 if X.dtype == self.torch.bfloat16 else bl.BL_F32
                assert bl.linear_fused(self.M_dec, m.K)
                arr[i] = bl._LinearProblem(X.data_ptr(), None if g is None else g.data_ptr(),
                                           self.P_dec[r][i].data_ptr(), self.g_dec[i].data_ptr(),
                                           self.Y_dec[i].data_ptr(), None, None,
                                           self.M_dec, m.N, m.K, dt, 1e-6)
            self.lin_dec_tables.append(arr)
        self.lin_dec_b3_tables = []
        for r in range(self.R_dec):
            arr = (bl._LinearProblem * n)()
            for i, m in enumerate(mats):
                X = self.X_dec[i]
                g = self.norms[i]
                dt = bl.BL_BF16 if X.dtype == self.torch.bfloat16 else bl.BL_F32
                arr[i] = bl._LinearProblem(X.data_ptr(), None if g is None else g.data_ptr(),
                                           self.B3_dec[r][i].data_ptr(), self.g_dec[i].data_ptr(),
                                           self.Y_dec[i].data_ptr(), None, None,
                                           self.M_dec, m.N, m.K, dt, 1e-6)
            self.lin_dec_b3_tables.append(arr)
        self.lin_dec_tiles_tables = []
        for r in range(self.R_dec):
            arr = (bl._LinearProblem * n)()
            for i, m in enumerate(mats):
                X = self.X_dec[i]
                g = self.norms[i]
                dt = bl.BL_BF16 if X.dtype == self.torch.bfloat16 else bl.BL_F32
                arr[i] = bl._LinearProblem(X.data_ptr(), None if g is None else g.data_ptr(),
                                           self.T_dec[r][i].data_ptr(), self.g_dec[i].data_ptr(),
                                           self.Y_dec[i].data_ptr(), None, None,
                                           self.M_dec, m.N, m.K, dt, 1e-6)
            self.lin_dec_tiles_tables.append(arr)
        import ctypes as C
        self._addr = C.addressof
        self.ws_ptr = self.ws.data_ptr()
        self.ws_bytes = self.ws.numel()

    # Work accounting (algorithmic, what the method must move or compute).
    def mixed_one_launch(self) -> bool:
        return mixed_one_launch(self.wl, self.M_pre, self.M_dec)

    def quantize_step(self, L, rp: int, stream) -> int:
        """The step's weight + activation quantization (weights into quad rows where the
        products read them there)."""
        fn = L.bitlinear_quantize_step_quad_rows if self.quad else L.bitlinear_quantize_step
        return fn(self._addr(self.wq_tables[rp]), self.count, self.ws_ptr, self.ws_bytes,
                  self._addr(self.aq_pre_tables[rp]), self.count, stream)

    def prefill(self, L, stream) -> int:
        """The step's prefill products as their own launch (on quad rows where they fit)."""
        fn = L.bitlinear_forward_quad_rows_grouped if self.quad else L.bitlinear_forward_grouped
        return fn(self._addr(self.fwd_pre_table), self.count, stream)

    def decode_leg(self, L, rd: int, stream) -> int:
        """The step's decode leg as its own launch (tiles or two-bit rows)."""
        if self.dec_tiles:
            return L.bitlinear_linear_tiles_grouped(self._addr(self.lin_dec_tiles_tables[rd]),
                                                    self.count, stream)
        return L.bitlinear_linear_grouped(self._addr(self.lin_dec_tables[rd]), self.count, stream)

    def prefill_ops(self) -> int:
        return sum(2 * self.M_pre * m.N * m.K for m in self.wl.matrices)

    def decode_bytes(self) -> int:
        # Packed weights, the raw activations (fp32 or bf16) and norm weights read, gamma, and
        # the fp32 outputs written.
        M = self.M_dec
        xb = 2 if self.wl.x_dtype == "bf16" else 4
        return sum(m.N * m.K // 4 + M * m.K * xb + (4 * m.K if m.norm else 0) + 4 + 4 * M * m.N
                   for m in self.wl.matrices)

    def decode_b3_bytes(self) -> int:
        M = self.M_dec
        xb = 2 if self.wl.x_dtype == "bf16" else 4
        return sum(m.N * self.bl.b3_row_bytes(m.K) + M * m.K * xb + (4 * m.K if m.norm else 0) + 4 + 4 * M * m.N
                   for m in self.wl.matrices)

    def prefill_bytes(self) -> int:
        # What the prefill product must move: int8 activations, packed weights, scales, gamma
        # and the fp32 outputs.
        M = self.M_pre
        return sum(M * m.K + m.N * m.K // 4 + 4 * M + 4 + 4 * M * m.N for m in self.wl.matrices)

    def weight_quant_bytes(self) -> int:
        if self.W_pre is None:
            return 0
        return sum(4 * m.N * m.K + m.N * m.K // 4 + 4 for m in self.wl.matrices)

    def act_quant_bytes(self, M: int) -> int:
        xb = 2 if self.wl.x_dtype == "bf16" else 4
        return sum(M * m.K * xb + M * m.K + 4 * M + (4 * m.K if m.norm else 0) for m in self.wl.matrices)

    def step(self, i: int, stream, ev=None):
        """Enqueue one step; `ev` (dict of event lists) brackets each launch group."""
        L = self.bl.lib()
        rp = i % self.R_pre
        rd = i % self.R_dec
        n = self.count

        def mark(key):
            if ev is not None:
                e = self.torch.cuda.Event(enable_timing=True)
                e.record()
                ev.setdefault(key, []).append(e)

        mark("t0")
        if self.wq_tables:
            # Weight quantization and the prefill activations' quantization in one call: the
            # gamma pass and the activation codes share a launch, the pack pass follows.
            rc = self.quantize_step(L, rp, stream)
        else:
            rc = L.bitlinear_quantize_acts_grouped(self._addr(self.aq_pre_tables[rp]), n, stream)
        assert rc == 0, rc
        mark("t_aq")
        if self.mixed_one_launch():
            # The prefill products and the decode leg in one launch (a mixed batch): the decode
            # blocks fill the compute units the products' last tiles leave idle.
            rc = L.bitlinear_forward_mixed(self._addr(self.fwd_pre_ex_table), n,
                                           self._addr(self.lin_dec_tables[rd]), n, stream)
            assert rc == 0, rc
        else:
            # 128 x 256 product tiles: the products, then the decode leg (the two launches the
            # mixed call makes for such a batch, made here so each can be bracketed).
            rc = self.prefill(L, stream)
            assert rc == 0, rc
            mark("t_pre")
            rc = self.decode_leg(L, rd, stream)
            assert rc == 0, rc
        mark("t_mix")

    def launch_only(self, key: str, i: int, stream):
        """One launch group of the step by itself (same tables as in the step)."""
        L = self.bl.lib()
        n = self.count
        if key == "prefill_gemm":
            rc = self.prefill(L, stream)
        elif key == "weight_and_act_quant":
            rc = self.quantize_step(L, i % self.R_pre, stream)
        elif key == "prefill_and_decode":
            if self.mixed_one_launch():
                rc = L.bitlinear_forward_mixed(self._addr(self.fwd_pre_ex_table), n,
                                               self._addr(self.lin_dec_tables[i % self.R_dec]), n, stream)
            else:       # the step's two launches
                rc = self.prefill(L, stream)
                assert rc == 0, rc
                rc = self.decode_leg(L, i % self.R_dec, stream)
        elif key == "decode_linear":
            rc = self.decode_leg(L, i % self.R_dec, stream)
        elif key == "decode_linear_rows":
            rc = L.bitlinear_linear_grouped(self._addr(self.lin_dec_tables[i % self.R_dec]), n, stream)
        elif key == "decode_linear_b3":
            rc = L.bitlinear_linear_b3_grouped(self._addr(self.lin_dec_b3_tables[i % self.R_dec]), n, stream)
        elif key == "act_quant_prefill":
            rc = L.bitlinear_quantize_acts_grouped(self._addr(self.aq_pre_tables[i % self.R_pre]), n, stream)
        elif self.quad:
            # Weight quantization alone, into the quad-row layout (the step call without
            # activations).
            rc = L.bitlinear_quantize_step_quad_rows(self._addr(self.wq_tables[i % self.R_pre]), n,
                                                     self.ws_ptr, self.ws_bytes, None, 0, stream)
        else:
            rc = L.bitlinear_quantize_weights_grouped(self._addr(self.wq_tables[i % self.R_pre]), n,
                                                       self.ws_ptr, self.ws_bytes, stream)
        assert rc == 0, rc


def isolated_ms(torch, setup: Setup, key: str, reps: int, loops: int = 5) -> float:
    """Duration of one launch group run alone, back to back: the median over `loops` timed
    replays of a HIP graph of `reps` launches (rotating through the input copies), divided by
    `reps`.  The graph keeps the host's per-launch cost (several us, as long as the shortest
    kernels here) out of the figure; events on the replay stream."""
    s_ = torch.cuda.Stream()
    with torch.cuda.stream(s_):
        for i in range(3):
            setup.launch_only(key, i, s_.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s_):
        for i in range(reps):
            setup.launch_only(key, i, s_.cuda_stream)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(loops)]
    with torch.cuda.stream(s_):
        graph.replay()
        for s, e in evs:
            s.record(s_)
            graph.replay()
            e.record(s_)
    torch.cuda.synchronize()
    return float(np.median([s.elapsed_time(e) for s, e in evs])) / reps


def interval_ms(ev, a, b):
    xs = [s.elapsed_time(e) for s, e in zip(ev[a], ev[b])]
    return float(np.mean(xs)) if xs else float("nan")


# Kernel name fragment -> (roofline key, source file).  (The decode leg quantizes its
# activations inside decode_kernel, so every act_quant launch belongs to the prefill leg.)
KERNELS = {
    "mixed_kernel": ("prefill_and_decode", "mixed.hip+prefill_core.hpp+decode_core.hpp+common.hpp"),
    "prefill_kernel": ("prefill_gemm", "prefill.hip+prefill_core.hpp+common.hpp"),
    "gemv_kernel": ("decode_linear", "gemv.hip+decode_core.hpp+common.hpp"),
    "decode_kernel": ("decode_linear", "decode.hip+decode_core.hpp+common.hpp"),
    "act_quant": ("act_quant_prefill", "quant.hip+common.hpp"),
    "gamma_partial_kernel": ("weight_quant", "quant.hip+common.hpp"),
    "gamma_act_kernel": ("gamma_and_act_quant", "quant.hip+common.hpp"),
    "quant_pack_kernel": ("weight_quant", "quant.hip+common.hpp"),
    "sample_kernel": ("weight_quant", "quant.hip+common.hpp"),
    "one_read_pass_kernel": ("weight_quant", "quant.hip+common.hpp"),
    "one_read_fix_kernel": ("weight_quant", "quant.hip+common.hpp"),
    "fix_act_kernel": ("fix_and_act_quant", "quant.hip+common.hpp"),
}

# Derived per-kernel figures from hardware counters (per dispatch, averaged over dispatches).
# `cyc` = GPU-active cycles of one XCD (GRBM_GUI_ACTIVE is summed over the XCDs); SQ_WAVE_CYCLES
# and SQ_WAIT_INST_ANY count in units of four cycles; MFMA instructions are among the VALU
# instructions SQ_INSTS_VALU counts.
COUNTER_FIGURES = [
    ("MFMA busy (% of SIMD-cycles)",
     lambda c, simds, cyc: 100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * simds)),
    ("VALU instructions per MFMA (MFMA included)", lambda c, simds, cyc: c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"]),
    ("LDS instructions per MFMA", lambda c, simds, cyc: c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"]),
    ("waves waiting (% of wave time)", lambda c, simds, cyc: 100.0 * c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]),
    ("mean waves resident per CU", lambda c, simds, cyc: 4.0 * c["SQ_WAVE_CYCLES"] / (cyc * simds / 4)),
    ("LDS bank-conflict cycles per LDS instruction",
     lambda c, simds, cyc: c["SQ_LDS_BANK_CONFLICT"] / c["SQ_ACTIVE_INST_LDS"]),
    ("LDS bank-conflict cycles (% of CU-cycles)",
     lambda c, simds, cyc: 100.0 * c["SQ_LDS_BANK_CONFLICT"] / (cyc * simds / 4)),
    ("vector-memory reads per wave", lambda c, simds, cyc: c["SQ_INSTS_VMEM_RD"] / c["SQ_WAVES"]),
    ("vector-memory writes per wave", lambda c, simds, cyc: c["SQ_INSTS_VMEM_WR"] / c["SQ_WAVES"]),
    ("L2 hit rate (%)", lambda c, simds, cyc: 100.0 * c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])),
    ("TA busy (% of cycles, mean over TAs)", lambda c, simds, cyc: 100.0 * c["TA_BUSY_avr"] / cyc),
]


def summarize_counters(paths, simds: int, xcds: int) -> str:
    """Markdown table of COUNTER_FIGURES per library kernel from rocprofv3 --pmc CSV files
    (counter_collection.csv; one file per counter pass of the same command)."""
    import csv
    from collections import defaultdict
    sums = defaultdict(lambda: defaultdict(float))   # kernel -> counter -> sum over dispatches
    dispatches = defaultdict(lambda: defaultdict(set))
    for path in paths:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            frag = next((f for f in KERNELS if f in name), None)
            if frag is None:
                continue
            key = name.split("(")[0].replace("void ", "")
            sums[key][r["Counter_Name"]] += float(r["Counter_Value"])
            dispatches[key][r["Counter_Name"]].add((path, r["Dispatch_Id"]))
    lines = ["| kernel | dispatches | " + " | ".join(n for n, _ in COUNTER_FIGURES) + " |",
             "|---|---|" + "---|" * len(COUNTER_FIGURES)]
    for key in sorted(sums):
        c = {k: v / max(1, len(dispatches[key][k])) for k, v in sums[key].items()}
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        vals = []
        for _, f in COUNTER_FIGURES:
            try:
                vals.append(f"{f(c, simds, cyc):.3g}")
            except (KeyError, ZeroDivisionError):
                vals.append("")
        n = max(len({i for _, i in d}) for d in dispatches[key].values())
        lines.append(f"| `{key}` | {n} | " + " | ".join(vals) + " |")
    return "\n".join(lines)


def summarize_pmc(fetch_csv: str, write_csv: str, workload: str, command: str) -> dict:
    """Per-launch HBM bytes of each kernel, scaled by a plain 256 MiB device copy."""
    import csv
    from collections import defaultdict
    wlw = workloads.WORKLOADS[workload]
    tiles_leg = decode_on_tiles(wlw, max(wlw.token_counts))

    def per_dispatch(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            name, grid = r["Kernel_Name"], int(r["Grid_Size"])
            prev = out.get(key, (name, grid, 0.0))
            out[key] = (name, grid, prev[2] + float(r["Counter_Value"]))
        return out

    fetch = per_dispatch(fetch_csv, "FETCH_SIZE")
    write = per_dispatch(write_csv, "WRITE_SIZE")
    copy_bytes = 256 * 1024 * 1024

    def calib(d):
        # The calibration copy is the process's first device copy (it runs before the setup
        # clones any input tensor).
        first_copy = min(k for k, (n, g, v) in d.items() if "copyBuffer" in n)
        return copy_bytes / (d[first_copy][2] * 1024.0)

    f_fetch, f_write = calib(fetch), calib(write)

    def by_kernel(d, factor):
        acc = defaultdict(list)
        for name, grid, kib in d.values():
            for frag, (key, src) in KERNELS.items():
                if frag in name:
                    if frag == "gemv_kernel":
                        lay = gemv_layout(name)       # the one-token kernel: which weight layout
                        if lay == "b3":
                            key = "decode_linear_b3"
                        elif (lay == "tiles") != tiles_leg:
                            key = "decode_linear_rows" if lay == "rows" else "decode_linear_tiles"
                    acc[(key, src)].append((name, kib * 1024.0 * factor))
                    break
        return acc

    fk, wk = by_kernel(fetch, f_fetch), by_kernel(write, f_write)
    kernels = {}
    def per_call(vals):
        # A call may be several kernels (weight quantization: gamma pass + pack pass, or sample +
        # pass + fix-up; activation quantization: wave and block kernels): the sum over the
        # call's kernels of each kernel's mean bytes per dispatch.
        by_name = defaultdict(list)
        for name, v in vals:
            by_name[name].append(v)
        return (sum(float(np.mean(v)) for v in by_name.values()),
                min(len(v) for v in by_name.values()), len(by_name))

    for (key, src), vals in fk.items():
        fetch_b, launches, nk = per_call(vals)
        wvals = wk.get((key, src), [])
        write_b = per_call(wvals)[0] if wvals else 0.0
        kernels[f"{key}@{workload}"] = {"kernel": key, "source": src, "source_sha": source_hash(src),
                                        "workload": workload, "fetch_scale": round(f_fetch, 4),
                                        "write_scale": round(f_write, 4),
                        "launches": launches, "kernels_per_call": nk,
                        "fetch_bytes_per_launch": round(fetch_b),
                        "write_bytes_per_launch": round(write_b),
                        "bytes_per_launch": round(fetch_b + write_b)}
    return {"command": command, "copy_calibration_bytes": copy_bytes,
            "fetch_scale": f_fetch, "write_scale": f_write, "kernels": kernels}


def load_traffic():
    """HBM traffic per launch from committed counter runs, if the kernel sources still match."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    out = {}
    for r in rec.get("kernels", {}).values():
        if r.get("source_sha") == source_hash(r["source"]) and r.get("workload"):
            out[(r["kernel"], r["workload"])] = r
    return out


def host_cores() -> int:
    """Host CPUs this process may run on (its affinity mask), capped at 16: the CPU share one
    GPU's process gets on the benchmark host."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(setup: Setup, budget_s: float):
    """Time the CPU oracle on a bounded sample of the step, twice: on one thread (the oracle as
    written), and on every host core the process may use, with the step's independent pieces
    (weight tensors; blocks of token rows of each product) spread over a thread pool.  The
    oracle itself stays single-threaded: each task is one call into it, and ctypes releases
    the interpreter lock for the call's duration."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    orc = oracle.get()
    wl = setup.wl
    h = setup.host
    mats = wl.matrices
    bf16 = wl.x_dtype == "bf16"
    macs = sum(m.N * m.K for m in mats)
    rate_guess = 1.4e9  # MAC/s of the oracle's scalar loop on a current x86 core
    cores = host_cores()

    def norm(i):
        return workloads.norm_weight(wl, i) if mats[i].norm else None

    def quantize_weight(i):
        if h["W"] is not None:
            P, g, codes = orc.quantize_weights(h["W"][i])
            return P, g, codes
        C = workloads.weight_codes(wl, i)
        return orc.pack(C), np.float32(wl.code_gamma), C

    def rows(i, X, codes, gamma):
        q, s = orc.quantize_acts(X, norm(i), 1e-6, bf16=bf16)
        return orc.epilogue(orc.matmul(q, codes), s, gamma)

    # One thread: every weight tensor, a sample of the prefill tokens, the decode token.
    M_s = int(max(1, min(setup.M_pre, round(0.5 * budget_s * rate_guess / macs))))
    t0 = time.perf_counter()
    packed = [quantize_weight(i) for i in range(len(mats))]
    t_w = time.perf_counter() - t0
    t1 = time.perf_counter()
    for i in range(len(mats)):
        rows(i, h["X_pre"][i][:M_s], packed[i][2], packed[i][1])
    t_pre = time.perf_counter() - t1
    t2 = time.perf_counter()
    for i in range(len(mats)):
        rows(i, h["X_dec"][i], packed[i][2], packed[i][1])
    t_dec = time.perf_counter() - t2
    step_1 = t_w + t_pre * (setup.M_pre / M_s) + t_dec

    # All cores: weight tensors in parallel, then blocks of token rows of every product.
    M_a = int(max(cores, min(setup.M_pre, M_s * cores)))
    blk = -(-M_a // cores)
    with ThreadPoolExecutor(max_workers=cores) as pool:
        t3 = time.perf_counter()
        packed_a = list(pool.map(quantize_weight, range(len(mats))))
        t_wa = time.perf_counter() - t3
        t4 = time.perf_counter()
        futs = [pool.submit(rows, i, h["X_pre"][i][r0:min(M_a, r0 + blk)], packed_a[i][2], packed_a[i][1])
                for i in range(len(mats)) for r0 in range(0, M_a, blk)]
        for f in futs:
            f.result()
        t_pa = time.perf_counter() - t4
        t5 = time.perf_counter()
        list(pool.map(lambda i: rows(i, h["X_dec"][i], packed_a[i][2], packed_a[i][1]), range(len(mats))))
        t_da = time.perf_counter() - t5
    step_a = t_wa + t_pa * (setup.M_pre / M_a) + t_da

    def sample(M_n):
        if M_n == setup.M_pre:
            return (f"one full step ({len(mats)} matrices: weight quantization, {setup.M_pre}-token "
                    "prefill, 1-token decode)")
        return (f"weight quantization of all {len(mats)} matrices, decode, and {M_n} of "
                f"{setup.M_pre} prefill tokens; prefill time scaled by {setup.M_pre / M_n:.1f} "
                "(a sampled extrapolation)")

    return {
        "value": setup.prefill_ops() / step_a / 1e12,
        "unit": "TOPS",
        "cores": cores,
        "kind": "oracle",
        "sample": sample(M_a),
        "seconds_measured": round(t_wa + t_pa + t_da, 3),
        "seconds_per_step": round(step_a, 3),
        "single_thread": {"value": setup.prefill_ops() / step_1 / 1e12, "cores": 1,
                          "sample": sample(M_s), "seconds_measured": round(t_w + t_pre + t_dec, 3),
                          "seconds_per_step": round(step_1, 3)},
        "parallel_over": "weight tensors, then blocks of token rows of each product "
                         "(one oracle call per task, a thread pool of `cores` workers)",
        "host_cpus_visible": os.cpu_count(),
        "cpu": cpu_model(),
    }


def copy_calibration(torch):
    """A plain device-to-device copy of a known size, for scaling HBM counters."""
    n = 256 * 1024 * 1024
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return n


def layer_bench(torch, bl, wl: workloads.Workload, M_pre: int, rotate_bytes: float, reps: int):
    """The workload's projections assembled into one transformer layer's BitLinear sub-graph
    (bit_gemm_02_amd.layer), timed at one token and at the prefill token count.  Distinct
    weight copies (about `rotate_bytes` in all) run one after another from a replayed HIP
    graph, so every layer reads its weights from HBM; activation buffers are shared."""
    from bit_gemm_02_amd import layer as L
    act = {"swiglu": bl.ACT_SWIGLU, "relu2": bl.ACT_RELU2}[wl.ffn]
    mats = {m.name: (i, m) for i, m in enumerate(wl.matrices)}
    if not {"o", "up", "down"} <= set(mats):
        raise SystemExit(f"{wl.key} is not a layer set (needs o, up and down projections)")
    if wl.weights == "fp32":
        names = list(mats)
        packed = bl.quantize_weights_grouped(
            [torch.from_numpy(workloads.weight_fp32(wl, mats[n][0])).cuda() for n in names])
        base = {n: pg for n, pg in zip(names, packed)}
    else:
        base = {}
        for n, (i, m) in mats.items():
            P = bl.pack_codes(torch.from_numpy(workloads.weight_codes(wl, i)).cuda())
            base[n] = (P, torch.full((1,), wl.code_gamma, device="cuda"))
    d = mats["down"][1].N
    norms = {}
    for j, (key, K) in enumerate((("attn", d), ("o", mats["o"][1].K), ("ffn", d),
                                  ("down", mats["down"][1].K))):
        g = np.float32(1) + workloads.gaussian((K,), (wl.index, 70 + j), 0.1)
        norms[key] = torch.from_numpy(g).cuda()
    w_bytes = sum(P.numel() * 4 for P, _ in base.values())
    R = int(max(1, min(1024, np.ceil(rotate_bytes / w_bytes))))
    layers = [L.LayerWeights(packed={n: P.clone() for n, (P, _) in base.items()},
                             gamma={n: g for n, (_, g) in base.items()}, norms=norms, act=act)
              for _ in range(R)]
    out = {"layer_copies": R, "ffn": wl.ffn, "projections": sorted(base)}
    for M in (1, M_pre):
        chains = [L.LayerChain(layers[0], M)]
        chains += [L.LayerChain(w, M, like=chains[0]) for w in layers[1:]]
        c0 = chains[0]
        c0.x.copy_(torch.from_numpy(workloads.gaussian((M, d), (wl.index, 80, M), 1.0)))
        c0.attn.copy_(torch.from_numpy(workloads.gaussian(tuple(c0.attn.shape), (wl.index, 81, M), 1.0)))
        s_ = torch.cuda.Stream()
        with torch.cuda.stream(s_):
            for c in chains[:3]:
                c(s_.cuda_stream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s_):
            for c in chains:
                c(s_.cuda_stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(s_):
            graph.replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s_)
            for _ in range(reps):
                graph.replay()
            e1.record(s_)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * R)
        ops = c0.ops()
        # Bytes a layer must move at least: packed weights, gammas, norm weights, the layer
        # input, the attention output and the layer output (intermediates not counted).
        nbytes = (w_bytes + 4 * len(base) + sum(4 * g.numel() for g in norms.values())
                  + 4 * M * (2 * d + c0.attn.shape[1]))
        key = "decode" if M == 1 else "prefill"
        out[key] = {"tokens": M, "us_per_layer": round(us, 3), "launches_per_layer": len(c0._calls),
                    "tokens_per_s_per_layer": round(M / (us * 1e-6), 1),
                    "tops": round(ops / (us * 1e-6) / 1e12, 2),
                    "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                    "bytes": nbytes, "ops": ops}
        del chains, graph
        torch.cuda.synchronize()
    return out


BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published (no sparsity)


def measured_peaks(torch, bl) -> dict:
    """What this GPU attains, from the library's calibration kernels, run once outside any timed
    region: a plain 16-byte-load read stream over 2 GiB (HBM, well past the 256 MB last-level
    cache) and loops of independent int8 and bf16 matrix-unit operations on every compute unit
    (at the clock the matrix units actually run at).  The rooflines are quoted against these
    beside the published peaks."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    sums = torch.empty(256 * 4 * cus, dtype=torch.int32, device="cuda")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps * 1e-3          # seconds per call

    hbm = buf.numel() / timed(lambda: bl.calib_stream(buf, out), 5) / 1e9
    iters = 4096
    ops = {k: bl.calib_mfma(k, iters, 4 * cus, sums) for k in (bl.CALIB_INT8, bl.CALIB_BF16)}
    int8 = ops[bl.CALIB_INT8] / timed(lambda: bl.calib_mfma(bl.CALIB_INT8, iters, 4 * cus, sums), 3) / 1e12
    bf16 = ops[bl.CALIB_BF16] / timed(lambda: bl.calib_mfma(bl.CALIB_BF16, iters, 4 * cus, sums), 3) / 1e12
    del buf
    return {"hbm_read_GBps": round(hbm, 1), "int8_mfma_TOPS": round(int8, 1),
            "bf16_mfma_TFLOPS": round(bf16, 1),
            "how": "bitlinear_calib_stream over 2 GiB; bitlinear_calib_mfma, 4 blocks of 4 waves "
                   "per compute unit, 8 independent accumulators per wave, 4096 iterations"}


def graph_ms(torch, fn, reps: int) -> float:
    """Average time of fn(stream) replayed from a captured HIP graph (events on its stream)."""
    s_ = torch.cuda.Stream()
    with torch.cuda.stream(s_):
        fn(s_.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s_):
        for _ in range(reps):
            fn(s_.cuda_stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(s_):
        graph.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s_)
        for _ in range(3):
            graph.replay()
        e1.record(s_)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (3 * reps)


def train_bench(torch, bl, wl: workloads.Workload, M: int, reps: int):
    """The workload's projections as one grouped call per training-side product at M tokens:
    the weight-only forward (fp32 and bf16 activations), the input gradient (fp32 dY), the
    weight gradient with the soft STE scale, and the transposed packing of every matrix.
    Inputs are seeded and resident; each product is timed from a replayed graph."""
    mats = wl.matrices
    dev = "cuda"
    g = torch.full((1,), wl.code_gamma, device=dev)
    Ps, Wts, Ws = [], [], []
    for i, m in enumerate(mats):
        C = torch.from_numpy(workloads.ternary((m.N, m.K), (wl.index, 90, i), wl.code_mix)).to(dev)
        Ps.append(bl.pack_codes(C))
        Wts.append(bl.transpose_packed(Ps[-1]))
        Ws.append(torch.from_numpy(workloads.gaussian((m.N, m.K), (wl.index, 91, i), wl.w_sigma)).to(dev))
    X = [torch.from_numpy(workloads.gaussian((M, m.K), (wl.index, 92, i), 1.0)).to(dev) for i, m in enumerate(mats)]
    Xb = [x.to(torch.bfloat16) for x in X]
    dY = [torch.from_numpy(workloads.gaussian((M, m.N), (wl.index, 93, i), 1.0)).to(dev) for i, m in enumerate(mats)]
    Y = [torch.empty((M, m.N), device=dev) for m in mats]
    dX = [torch.empty((M, m.K), device=dev) for m in mats]
    dW = [torch.empty((m.N, m.K), device=dev) for m in mats]
    qs = [bl.quantize_acts(x) for x in X]
    L = bl.lib()
    import ctypes
    tabs = {}
    arr = (bl._WonlyProblem * len(mats))()
    arrb = (bl._WonlyProblem * len(mats))()
    gi = (bl._GradInputProblem * len(mats))()
    gw = (bl._GradWeightProblem * len(mats))()
    for i, m in enumerate(mats):
        arr[i] = bl._WonlyProblem(X[i].data_ptr(), Ps[i].data_ptr(), g.data_ptr(), Y[i].data_ptr(), M, m.N, m.K, bl.BL_F32)
        arrb[i] = bl._WonlyProblem(Xb[i].data_ptr(), Ps[i].data_ptr(), g.data_ptr(), Y[i].data_ptr(), M, m.N, m.K, bl.BL_BF16)
        gi[i] = bl._GradInputProblem(dY[i].data_ptr(), Wts[i].data_ptr(), g.data_ptr(), dX[i].data_ptr(), M, m.N, m.K, bl.BL_F32)
        gw[i] = bl._GradWeightProblem(dY[i].data_ptr(), qs[i][0].data_ptr(), qs[i][1].data_ptr(), Ws[i].data_ptr(),
                                      g.data_ptr(), dW[i].data_ptr(), M, m.N, m.K, bl.STE_SOFT, 2.0)
    n = len(mats)

    def call(fn, a):
        return lambda st: bl._check(fn.__name__, fn(ctypes.addressof(a), n, st))

    def transpose_all(st):
        for i, m in enumerate(mats):
            bl._check("transpose", L.bitlinear_transpose_packed(Ps[i].data_ptr(), m.N, m.K, Wts[i].data_ptr(), st))

    flops = sum(2 * M * m.N * m.K for m in mats)
    packed = sum(m.N * m.K // 4 for m in mats)
    peaks = measured_peaks(torch, bl)
    bf16_meas = peaks["bf16_mfma_TFLOPS"]
    out = {"tokens": M, "matrices": [f"{m.name} {m.K}->{m.N}" for m in mats], "flops_per_product": flops,
           "measured_peaks": peaks}
    for key, fn, f32 in (("forward_wonly_f32", call(L.bitlinear_forward_wonly_grouped, arr), True),
                         ("forward_wonly_bf16", call(L.bitlinear_forward_wonly_grouped, arrb), False),
                         ("grad_input_f32", call(L.bitlinear_grad_input_grouped, gi), True),
                         ("grad_weight_soft", call(L.bitlinear_grad_weight_grouped, gw), True)):
        ms = graph_ms(torch, fn, reps)
        tf = flops / (ms * 1e-3) / 1e12
        out[key] = {"us": round(ms * 1e3, 2), "tflops": round(tf, 1),
                    "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                    "mfma_per_product": 2 if f32 else 1,
                    "frac_attainable": round(tf * (2 if f32 else 1) / BF16_PEAK_TFLOPS, 4),
                    "frac_attainable_measured": round(tf * (2 if f32 else 1) / bf16_meas, 4)}
    ms = graph_ms(torch, transpose_all, reps)
    out["transpose_packed"] = {"us": round(ms * 1e3, 2), "bytes": 2 * packed,
                               "gbps": round(2 * packed / (ms * 1e-3) / 1e9, 1)}
    return out


def main():
    args = parse()
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.simds, args.xcds))
        return
    if args.summarize_pmc:
        cmd = ("rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- python3 "
               f"bench.py --workload {args.workload} --steps 3 --warmup 1 --no-cpu-baseline "
               "--min-warmup-s 0.2 --copy-calibration")
        rec = summarize_pmc(*args.summarize_pmc, args.workload, cmd)
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        old = {}
        if os.path.exists(TRAFFIC_FILE):
            old = json.load(open(TRAFFIC_FILE)).get("kernels", {})
        # Keep other workloads' records; replace this workload's.
        merged = {k: v for k, v in old.items() if v.get("workload") != args.workload}
        merged.update(rec["kernels"])
        rec["kernels"] = merged
        json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
        print(json.dumps(rec, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU sharding "
              "of this path is described in DESIGN.md and is not launched.", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_gemm_02_amd as bl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = workloads.WORKLOADS[args.workload]
    M_pre = args.prefill_tokens or max(wl.token_counts)
    if args.train:
        rec = train_bench(torch, bl, wl, M_pre, max(2, args.steps // 10))
        print(json.dumps({"metric": "BitLinear training-side products: TFLOP/s vs bf16 MFMA peak",
                          "workload": wl.key, "data": "synthetic", "n_gpus": 1, **rec}), flush=True)
        return
    if args.layer:
        rec = layer_bench(torch, bl, wl, M_pre, args.rotate_bytes, max(1, args.steps // 10))
        print(json.dumps({"metric": "BitLinear layer chain: us per layer (decode, prefill)",
                          "workload": wl.key, "data": "synthetic", "n_gpus": 1, **rec}), flush=True)
        return
    if args.copy_calibration:
        copy_calibration(torch)     # first device work of the process (see summarize_pmc)
    setup = Setup(torch, bl, wl, M_pre, args.rotate_bytes)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    # Warm-up: at least `warmup` steps and at least `min_warmup_s` seconds of them.  On a GPU
    # that was idle, the Qwen3-4B step ran 1.087 ms per step over the first ~20 ms of this load
    # and 1.005 ms once it had run for ~100 ms (the same process, the same steps); 5 steps are
    # 5 ms of it.
    warm = 0
    t_warm0 = time.perf_counter()
    while warm < args.warmup or time.perf_counter() - t_warm0 < args.min_warmup_s:
        for _ in range(max(1, args.warmup)):
            setup.step(warm, sptr)
            warm += 1
        torch.cuda.synchronize()

    # Timed region: exactly `steps` steps, bracketed by synchronizations.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        setup.step(warm + i, sptr)
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall0) * 1e3 / args.steps
    ms_per_step = start.elapsed_time(end) / args.steps

    # Per-launch durations, two ways, both outside the timed region: (a) the same steps again
    # with events around every launch group (includes the dispatch gap each launch pays inside
    # the step); (b) each launch group alone, back to back from a replayed graph (what a
    # kernel trace reports as its duration; used for the roofline figures).
    ev = {}
    for i in range(args.steps):
        setup.step(warm + args.steps + i, sptr, ev)
    torch.cuda.synchronize()
    in_step = {
        ("weight_and_act_quant" if setup.wq_tables else "act_quant_prefill"): interval_ms(ev, "t0", "t_aq"),
        "prefill_and_decode": interval_ms(ev, "t_aq", "t_mix"),
    }
    if "t_pre" in ev:
        in_step["prefill_gemm"] = interval_ms(ev, "t_aq", "t_pre")
        in_step["decode_linear"] = interval_ms(ev, "t_pre", "t_mix")
    ms_with_events = interval_ms(ev, "t0", "t_mix")
    # Isolated launches: the step's own, plus the product and the decode leg each alone.
    ms = {k: isolated_ms(torch, setup, k, args.steps)
          for k in set(in_step) | {"prefill_gemm", "decode_linear", "act_quant_prefill"} |
          ({"weight_quant"} if setup.wq_tables else set()) |
          ({"decode_linear_rows"} if setup.dec_tiles else set())}
    ms_b3 = isolated_ms(torch, setup, "decode_linear_b3", args.steps)
    peaks = measured_peaks(torch, bl)

    ops = setup.prefill_ops()
    pre_bytes = setup.prefill_bytes()
    dec_bytes = setup.decode_bytes()
    wq_bytes = setup.weight_quant_bytes()
    aq_bytes = setup.act_quant_bytes(M_pre)
    ridge = INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)          # ops per byte
    ai = ops / pre_bytes
    gemm_tops = ops / (ms["prefill_gemm"] * 1e-3) / 1e12
    gemm_gbps = pre_bytes / (ms["prefill_gemm"] * 1e-3) / 1e9
    attainable = min(INT8_PEAK_TOPS, ai * HBM_PEAK_GBPS / 1e3)     # TOPS
    dec_gbps = dec_bytes / (ms["decode_linear"] * 1e-3) / 1e9

    def hbm(nbytes, key, what):
        a = nbytes / (ms[key] * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBPS, "peak_measured": peaks["hbm_read_GBps"],
                "frac_measured": a / peaks["hbm_read_GBps"], "us_per_launch": ms[key] * 1e3,
                "us_per_launch_in_step": in_step[key] * 1e3 if key in in_step else None,
                "algorithmic": what}

    pre_what = (f"{ops} int8 ops (2 M N K over {setup.count} products); {pre_bytes} bytes "
                f"(M K + N K / 4 + 4 M + 4 + 4 M N summed); {ai:.0f} ops/B vs ridge {ridge:.0f}")
    if ai < ridge:
        # Below the ridge the product is bound by HBM: measure it in bytes.
        pre_roof = hbm(pre_bytes, "prefill_gemm", pre_what)
    else:
        pre_roof = {"bound": "mfma", "achieved": gemm_tops, "peak": INT8_PEAK_TOPS,
                    "unit": "TFLOP/s", "frac": gemm_tops / INT8_PEAK_TOPS,
                    "peak_measured": peaks["int8_mfma_TOPS"],
                    "frac_measured": gemm_tops / peaks["int8_mfma_TOPS"],
                    "us_per_launch": ms["prefill_gemm"] * 1e3,
                    "us_per_launch_in_step": (in_step["prefill_gemm"] * 1e3
                                              if "prefill_gemm" in in_step else None),
                    "algorithmic": pre_what}
    attainable_meas = min(peaks["int8_mfma_TOPS"], ai * peaks["hbm_read_GBps"] / 1e3)
    pre_roof.update({"tops": gemm_tops, "frac_int8_peak": gemm_tops / INT8_PEAK_TOPS,
                     "attainable_tops": attainable, "frac_attainable": gemm_tops / attainable,
                     "attainable_tops_measured": attainable_meas,
                     "frac_attainable_measured": gemm_tops / attainable_meas})
    rooflines = {
        "prefill_gemm": pre_roof,
        "decode_linear": hbm(dec_bytes, "decode_linear",
                             f"{dec_bytes} bytes (N K / 4 + M K x-bytes (+ 4 K norm) + 4 + 4 M N "
                             "summed; activation quantization fused; weights in the "
                             f"{'decode tile layout' if setup.dec_tiles else 'two-bit rows'})"),
        "act_quant_prefill": hbm(aq_bytes, "act_quant_prefill",
                                 f"{aq_bytes} bytes (M K x-bytes + M K + 4 M (+ 4 K norm) summed)"),
    }
    mix_bytes = pre_bytes + dec_bytes
    rooflines["prefill_and_decode"] = hbm(
        mix_bytes, "prefill_and_decode",
        f"{mix_bytes} bytes (the prefill products' {pre_bytes} and the decode leg's {dec_bytes}, "
        f"one launch); {ops} int8 ops; {ops / mix_bytes:.0f} ops/B vs ridge {ridge:.0f}")
    if "weight_and_act_quant" in ms:
        wa_bytes = wq_bytes + aq_bytes
        rooflines["weight_and_act_quant"] = hbm(
            wa_bytes, "weight_and_act_quant",
            f"{wa_bytes} bytes (the weight quantization's {wq_bytes} and the activation "
            f"quantization's {aq_bytes}; " +
            ("one read of W: the sample, the pass, the fix-up beside the activation rows longer "
             "than 4096 values, then the other activation rows)" if setup.one_read else
             "two reads of W: gamma pass + activation codes, then the pack pass)"))
    if "weight_quant" in ms:
        rooflines["weight_quant"] = hbm(wq_bytes, "weight_quant",
                                        f"{wq_bytes} bytes (4 N K + N K / 4 + 4 summed; one read "
                                        "of W is the minimum, " +
                                        ("which the one-read form reaches: sample, pass, fix-up)"
                                         if setup.one_read else "the two launches read it twice)"))
    # Dominant kernel = the step's largest single launch: the products' launch (with the decode
    # blocks when the mixed call shares one launch; the product alone where it cannot, with
    # 128 x 256 tiles).  The quantization call is two to four launches (one-read form: sample,
    # pass, fix-up + long rows, other rows; else gamma + activation codes, then the pack pass),
    # each shorter.
    fused = setup.mixed_one_launch()
    dom = "prefill_and_decode" if fused else "prefill_gemm"
    traffic = load_traffic()
    t = traffic.get((dom, wl.key))
    roof = dict(rooflines[dom])
    roof = {"kernel": dom, "bound": roof["bound"], "achieved": round(roof["achieved"], 2),
            "peak": roof["peak"], "unit": roof["unit"], "frac": round(roof["frac"], 4),
            "traffic": None if t is None else t["bytes_per_launch"],
            "peak_measured": roof["peak_measured"], "frac_measured": round(roof["frac_measured"], 4)}

    value = ops / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.key, "matrices": [f"{m.name} {m.K}->{m.N}" for m in wl.matrices],
                   "prefill_tokens": M_pre, "decode_tokens": 1,
                   "weights": wl.weights, "x_dtype": wl.x_dtype,
                   "rotation_copies": {"prefill": setup.R_pre, "decode": setup.R_dec}},
        "decode": {"gbps": round(dec_gbps, 2), "frac_hbm": round(dec_gbps / HBM_PEAK_GBPS, 4),
                   "bytes": dec_bytes, "us_linear": round(ms["decode_linear"] * 1e3, 3),
                   "layout": "tiles" if setup.dec_tiles else "rows",
                   **({"rows": {"us_linear": round(ms["decode_linear_rows"] * 1e3, 3),
                                "gbps": round(dec_bytes / (ms["decode_linear_rows"] * 1e-3) / 1e9, 2),
                                "note": "the same call on the two-bit rows [N][K/16]; the step's leg "
                                        "reads the decode tiles (same codes, packed once outside "
                                        "timing)"}} if setup.dec_tiles else {}),
                   "base3": {"us_linear": round(ms_b3 * 1e3, 3), "bytes": setup.decode_b3_bytes(),
                             "gbps": round(setup.decode_b3_bytes() / (ms_b3 * 1e-3) / 1e9, 2),
                             "speedup_vs_two_bit": round(ms["decode_linear"] / ms_b3, 3),
                             "note": "same codes in the base-3 layout (1.6 bits per weight), "
                                     "fused decode call; not part of the step"}},
        "prefill": {"weight_layout": "quad_rows" if setup.quad else "rows",
                    "gemm_tops": round(gemm_tops, 2), "frac_int8": round(gemm_tops / INT8_PEAK_TOPS, 4),
                    "gemm_gbps": round(gemm_gbps, 1), "ops_per_byte": round(ai, 1),
                    "frac_attainable": round(gemm_tops / attainable, 4),
                    "ops": ops, "us_gemm": round(ms["prefill_gemm"] * 1e3, 3),
                    "us_weight_quant": round(ms["weight_quant"] * 1e3, 3) if "weight_quant" in ms else None,
                    "weight_quant_form": (("one read (sample, pass with listed band, fix-up)"
                                           if setup.one_read else "two reads (gamma pass, pack pass)")
                                          if setup.W_pre is not None else None),
                    "us_act_quant": round(ms["act_quant_prefill"] * 1e3, 3),
                    "us_prefill_and_decode": round(ms["prefill_and_decode"] * 1e3, 3),
                    "us_weight_and_act_quant": round(ms["weight_and_act_quant"] * 1e3, 3) if "weight_and_act_quant" in ms else None,
                    "us_prefill_plus_decode_separate": round((ms["prefill_gemm"] + ms["decode_linear"]) * 1e3, 3)},
        "roofline": roof,
        "measured_peaks": peaks,
        "rooflines": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                      for k, v in rooflines.items()},
        "timing": {"ms_per_step_wall": round(wall_ms, 4),
                   "mixed_launch": "one launch" if fused else "two launches (128 x 256 product tiles)",
                   "ms_per_step_with_launch_events": round(ms_with_events, 4),
                   "schedule": "one stream, launches in step order: weight quantization, "
                               "activation quantization, then the prefill products and the decode "
                               "leg (one mixed launch where the products take 128 x 128 tiles). "
                               "Measured slower than one stream: three streams (weight quant "
                               "beside act quant, decode beside prefill), the decode leg alone on "
                               "a second stream, and on the Qwen3-4B set the quantization of later "
                               "projections on a second stream beside the products of earlier "
                               "ones (the product's 128 x 256 tile fills every register file) and "
                               "the decode leg on a second stream beside the quantization (no gain)"},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(setup, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
