"""Benchmark of the grouped 4-bit MoE layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config qwen235]

A step is one pass of the hot path over one batch of synthetic tokens:
gnf4_route -> gnf4_grouped_gemm (gate_up, rows gathered from the token
activations) -> gnf4_grouped_gemm (down, input already in routed order) ->
gnf4_combine (at T = 1 two launches: the routing fused into the gate_up GEMV,
the combine into the down GEMV). The default workload is the
Qwen3-235B-A22B-shaped layer, decode T = 1 and prefill T = 4096. Exactly K
consecutive steps are captured as HIP graphs (at most 256 steps per graph,
replayed back to back on one stream) and timed with HIP events on that
stream; successive steps rotate over input slots and over copies of the
layer's packed weights so that no step finds its weights in the 256 MB
Infinity Cache. The step time therefore does not depend on K.

Reported (one JSON line on stdout):
  value      decode packed-weight GB/s of the whole step (codes + scales of
             the experts the step routes to, both projections, / step time)
  roofline   the decode gate_up GEMM kernel: algorithmic packed bytes per
             launch / its mean duration from HIP events on the launch stream,
             beside the achievable read rate for the same bytes
             (gnf4_read_probe, a plain streaming read timed the same way)
  prefill    TFLOP/s of the prefill step and the roofline of its gate_up
             MFMA kernel (algorithmic flops 2*rows*N*K per launch)
  dequant_path  the same step through the dequantize-then-matmul path the
             pages compare against (bf16 decode of the routed experts to HBM,
             then library GEMMs), and the fused path's speed-up over it
  ffn_layer  the whole FFN layer step (router top-k from logits, gate_up with
             the SwiGLU epilogue, down on its bf16 output, combine) at the
             same T's
  streaming  decode steps with the packed experts in pinned host memory and
             an HBM cache of max(k, E/4) expert slots per projection: step
             time, experts and bytes streamed per step, the link ceilings, and
             the bytes / link + resident-step model
  cpu_baseline  the float64 CPU oracle (dequant + matmul + combine) timed on
             this host on one decode step of the same workload
Inputs are resident in device memory before timing starts.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--summarize", default=None, metavar="TITLE",
                    help="print a profile summary from rocprofv3 csv output (--trace, --pmc) "
                         "instead of benchmarking")
    ap.add_argument("--trace", nargs=2, action="append", default=[], metavar=("DIR", "CMD"),
                    help="a --kernel-trace output directory and the command that made it")
    ap.add_argument("--pmc", nargs=2, action="append", default=[], metavar=("DIR", "CMD"),
                    help="a --pmc output directory and the command that made it")
    ap.add_argument("--kernel", default=None,
                    help="with --summarize: the kernel (name substring) whose HBM traffic is "
                         "computed from FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--alg-bytes", type=int, default=None,
                    help="with --summarize: algorithmic bytes per launch of --kernel")
    ap.add_argument("--source", default="bit_mixture_experts_topk_amd/csrc/gemm.hip",
                    help="with --summarize: the source file of --kernel (its sha256 is recorded)")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen235")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dequant-path", action="store_true",
                    help="skip the dequantize-then-matmul comparison leg")
    ap.add_argument("--only", choices=["decode", "prefill", "backward", "streaming"], default=None,
                    help="run only the forward decode leg, the forward prefill leg, the "
                         "backward legs, or the host-RAM streaming leg")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--kernel-only", choices=["decode", "prefill"], default=None,
                    help="launch only the gate_up grouped GEMM of one step, --steps times "
                         "(for hardware-counter passes); prints no JSON")
    ap.add_argument("--proj", default=None, help="projection for --kernel-only (default gate_up): "
                    "gate_up runs gnf4_route_grouped_gemm, down gnf4_grouped_gemm_combine")
    ap.add_argument("--dx", action="store_true",
                    help="with --kernel-only: launch the input-gradient GEMM instead")
    return ap.parse_args()


def kernel_only(args):
    """One grouped-GEMM launch shape, repeated: the unit that counter passes
    measure. Launches rotate over copies of the projection's packed weights
    and over routing slots (token ids and activations), so that, as in the
    timed steps, a launch does not find its weights in the Infinity Cache."""
    import torch

    import synth
    from bit_mixture_experts_topk_amd import gnf4
    gnf4.lib()
    cfg = synth.CONFIGS[args.config]
    proj = cfg.proj(args.proj) if args.proj else cfg.projs[0]
    T = min(cfg.Ts) if args.kernel_only == "decode" else max(cfg.Ts)
    g = torch.Generator(device="cuda")
    g.manual_seed(17 * cfg.config_id + 1)
    pw = gnf4.empty_packed(cfg.fmt, cfg.E, proj.N, proj.K)
    W = torch.randn((cfg.E, proj.N, proj.K), generator=g, device="cuda") * 0.02
    gnf4.quantize(cfg.fmt, W, pw)
    del W
    per_launch = pw.nbytes() * min(1.0, T * cfg.k / cfg.E)
    copies = int(min(8, max(1, np.ceil(3 * MALL_BYTES / per_launch))))
    pws = [pw] + [type(pw)(pw.format, pw.E, pw.N, pw.K, pw.codes.clone(), pw.scales.clone(),
                           pw.scales2.clone() if pw.scales2 is not None else None)
                  for _ in range(copies - 1)]
    nslots = max(copies, 16 if T == 1 else 2)
    rows = T if proj.gather else T * cfg.k
    slots = []
    for i in range(nslots):
        ids, tw = synth.routing_inputs(cfg, T, seed=900 + i)
        X = torch.from_numpy(synth.activations(cfg, rows, proj.K, synth.T_X, 900 + i, T)
                             .view(np.int16)).cuda()
        ids_d = torch.from_numpy(ids).cuda()
        slots.append(dict(ids=ids_d, tw=torch.from_numpy(tw).cuda(), X=X, r=gnf4.route(ids_d, cfg.E)))
    Y = torch.empty((T * cfg.k, proj.N), dtype=torch.float32, device="cuda")
    out = torch.empty((T, proj.N), dtype=torch.float32, device="cuda")
    if args.dx:
        dY = torch.from_numpy(synth.grad_rows(cfg, T * cfg.k, proj.N, 0, T).view(np.int16)).cuda()
        dA = torch.empty((T * cfg.k, proj.K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for i in range(args.steps):
        sl, w = slots[i % nslots], pws[i % copies]
        if args.dx:
            gnf4.grouped_gemm_dx(w, dY, sl["r"], T, cfg.k, dA)
        elif proj.gather:                         # as the step runs it (routing fused in at T = 1)
            gnf4.route_grouped_gemm(sl["ids"], w, sl["X"], out=sl["r"], Y=Y)
        else:                                     # as the step runs it (combine fused in at T = 1)
            gnf4.grouped_gemm_combine(w, sl["X"], sl["r"], sl["tw"], T, cfg.k, out, Y=Y)
    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
    torch.cuda.synchronize()
    print("kernel-only %s %s %s%s T=%d x%d done" % (cfg.name, proj.name, args.kernel_only,
                                                    " dx" if args.dx else "", T, args.steps),
          file=sys.stderr, flush=True)


# ------------------------------------------------ rocprofv3 summaries

CALIB_COPY_BYTES = 1 << 30


def _csvs(d, suffix):
    import glob
    return sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))


def short_name(name):
    """A kernel's name without namespaces' argument lists: 'gnf4::x<1, 2>(...)' -> 'gnf4::x<1, 2>'."""
    name = name.replace("void ", "", 1) if name.startswith("void ") else name
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def trace_table(d):
    """Rows (kernel, grid, workgroup, lds, vgpr, calls, avg, min, p10, p50, p90 in us) of the
    dispatches in a rocprofv3 kernel-trace directory, by kernel and launch shape."""
    import csv
    groups = {}
    for f in _csvs(d, "kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]),
                   int(r["LDS_Block_Size"]), int(r["VGPR_Count"]) + int(r.get("Accum_VGPR_Count") or 0))
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            groups.setdefault(key, []).append(us)
    rows = []
    for key, v in groups.items():
        a = np.array(v)
        rows.append(key + (len(a), a.mean(), a.min(), np.percentile(a, 10), np.median(a),
                           np.percentile(a, 90)))
    rows.sort(key=lambda r: -r[5] * r[6])
    return rows


def pmc_table(d):
    """{(kernel, grid): {counter: [values per dispatch]}} of a --pmc directory."""
    import csv
    out = {}
    for f in _csvs(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
            out.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return out


def summarize(args):
    """The profile summary text: kernel-duration tables of the trace runs,
    per-dispatch counter means of the --pmc runs, and the HBM bytes per
    launch of --kernel from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by what the counter reads for the run's plain 1 GiB device
    copy (bench.py --calib-copy)."""
    import hashlib
    lines = ["# rocprofv3 summary: " + args.summarize, ""]
    for d, cmd in args.trace:
        lines += ["kernel trace command (from the repository root):", "  " + cmd, ""]
        lines.append("%-58s %9s %5s %6s %5s %6s %9s %9s %9s %9s %9s" % (
            "kernel", "grid", "wg", "lds", "vgpr", "calls", "avg_us", "min_us", "p10_us", "p50_us",
            "p90_us"))
        for r in trace_table(d):
            if not r[0].startswith("gnf4::"):
                continue
            lines.append("%-58s %9d %5d %6d %5d %6d %9.2f %9.2f %9.2f %9.2f %9.2f" % (
                r[0][:58], r[1], r[2], r[3], r[4], r[5], r[6], r[7], r[8], r[9], r[10]))
        lines.append("")
    traffic = {}
    for d, cmd in args.pmc:
        lines += ["counter pass (from the repository root):", "  " + cmd]
        tab = pmc_table(d)
        counters = sorted({c for v in tab.values() for c in v})
        for key in sorted(tab):
            if not key[0].startswith("gnf4::"):
                continue
            vals = ["%s %.6g" % (c, np.mean(tab[key][c])) for c in counters if c in tab[key]]
            n = max(len(v) for v in tab[key].values())
            lines.append("  %s grid %d (%d dispatches): %s" % (key[0], key[1], n, ", ".join(vals)))
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c not in counters:
                continue
            copies = [np.max(v[c]) for k, v in tab.items() if "copyBuffer" in k[0] and c in v]
            mine = [v[c] for k, v in tab.items() if args.kernel and args.kernel in k[0] and c in v]
            if not copies or not mine:
                continue
            calib = max(copies)
            factor = CALIB_COPY_BYTES / (calib * 1024.0)
            per = float(np.mean(np.concatenate(mine)))
            traffic[c] = per * 1024.0 * factor
            lines.append("  %s of %s: %.1f KiB/dispatch; the plain 1 GiB device copy: %.1f KiB -> "
                         "factor %.4f" % (c, args.kernel, per, calib, factor))
        lines.append("")
    if args.kernel and args.alg_bytes:
        lines.append("algorithmic bytes per launch of %s: %d" % (args.kernel, args.alg_bytes))
        if "FETCH_SIZE" in traffic and "WRITE_SIZE" in traffic:
            t = traffic["FETCH_SIZE"] + traffic["WRITE_SIZE"]
            lines.append("traffic_bytes_per_launch: %d" % int(round(t)))
            lines.append("traffic_over_algorithmic: %.3f" % (t / args.alg_bytes))
    import shlex
    lines += ["", "summary command (from the repository root):",
              "  python bench.py " + " ".join(shlex.quote(x) for x in sys.argv[1:])]
    if args.kernel:
        lines.append("kernel_source: %s" % args.source)
        lines.append("source_sha256: %s" % hashlib.sha256(open(os.path.join(ROOT, args.source), "rb")
                                                          .read()).hexdigest())
    print("\n".join(lines))


def packed_bytes_per_expert(pw):
    return pw.nbytes() // pw.E


class Layer:
    """Packed weights of one FFN layer (or the single projection of tiny)."""

    def __init__(self, torch, gnf4, cfg, seed=0):
        self.cfg = cfg
        self.projs = []
        g = torch.Generator(device="cuda")
        for pi, proj in enumerate(cfg.projs):
            g.manual_seed(1000 * seed + 17 * cfg.config_id + pi)
            pw = gnf4.empty_packed(cfg.fmt, cfg.E, proj.N, proj.K)
            if cfg.fmt == "nf4_dq":
                W = torch.randn((cfg.E, proj.N, proj.K), generator=g, device="cuda") * 0.02
                gnf4.quantize(cfg.fmt, W, pw)
                del W
            else:
                step = max(1, (1 << 28) // (proj.N * proj.K))   # experts per quantize call
                for e0 in range(0, cfg.E, step):
                    n = min(step, cfg.E - e0)
                    W = torch.randn((n, proj.N, proj.K), generator=g, device="cuda") * 0.02
                    gnf4.quantize_into(cfg.fmt, W, pw, e0)
                    del W
            self.projs.append(pw)
        torch.cuda.synchronize()

    def clone(self, torch):
        other = Layer.__new__(Layer)
        other.cfg = self.cfg
        other.projs = []
        for pw in self.projs:
            other.projs.append(type(pw)(pw.format, pw.E, pw.N, pw.K, pw.codes.clone(),
                                        pw.scales.clone(),
                                        pw.scales2.clone() if pw.scales2 is not None else None))
        return other

    def nbytes(self):
        return sum(pw.nbytes() for pw in self.projs)


class StepSlot:
    """Inputs, outputs and the captured graph of one step. ffn: the whole FFN
    layer (router top-k from logits, gate_up, SwiGLU, down on its output,
    combine) instead of route + both projections on standalone inputs."""

    def __init__(self, torch, gnf4, cfg, layer, T, seed, ffn=False):
        import synth
        k = cfg.k
        self.ffn = ffn
        if ffn:
            logits = synth.router_logits(cfg, T, seed=seed).astype(np.float32)
            self.logits = torch.from_numpy(logits).cuda()
            ids = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
            tw = np.zeros((T, k), dtype=np.float32)
        else:
            ids, tw = synth.routing_inputs(cfg, T, seed=seed)
        self.n_active = int(np.unique(ids).size)
        self.T = T
        self.ids = torch.from_numpy(ids).cuda()
        self.tw = torch.from_numpy(tw).cuda()
        first = cfg.projs[0]
        self.X = torch.from_numpy(synth.activations(cfg, T, first.K, synth.T_X, seed, T).view(np.int16)).cuda()
        self.layer = layer
        self.r = gnf4.route_buffers(T, k, cfg.E)
        self.r["topk_ids"] = torch.empty((T, k), dtype=torch.int32, device="cuda")
        self.r["topk_w"] = torch.empty((T, k), dtype=torch.float32, device="cuda")
        self.Y = [torch.empty((T * k, p.N), dtype=torch.float32, device="cuda") for p in cfg.projs]
        if ffn:
            self.H = torch.empty((T * k, cfg.inter), dtype=torch.int16, device="cuda")
        elif len(cfg.projs) > 1:
            down = cfg.projs[1]
            self.Xd = torch.from_numpy(synth.activations(cfg, T * k, down.K, synth.T_X_DOWN, seed, T)
                                       .view(np.int16)).cuda()
        self.out = torch.empty((T, cfg.projs[-1].N), dtype=torch.float32, device="cuda")

    def run(self, gnf4):
        cfg, T, k = self.layer.cfg, self.T, self.layer.cfg.k
        if self.ffn:
            # router top-k + routing + gate_up with SwiGLU, down + combine
            r, _ = gnf4.route_logits_grouped_gemm(self.logits, k, self.layer.projs[0], self.X,
                                                  out=self.r, H=self.H, swiglu=True)
            gnf4.grouped_gemm_combine(self.layer.projs[1], self.H, r, r["topk_w"], T, k, self.out,
                                      Y=self.Y[1])
            return
        # route + first projection, second projection + combine: one launch
        # each for a single token (the separate calls otherwise)
        r, _ = gnf4.route_grouped_gemm(self.ids, self.layer.projs[0], self.X, out=self.r, Y=self.Y[0])
        if len(self.layer.projs) > 1:
            gnf4.grouped_gemm_combine(self.layer.projs[1], self.Xd, r, self.tw, T, k, self.out,
                                      Y=self.Y[1])
        else:
            gnf4.combine(self.Y[0], r["inv"], self.tw, T, k, self.out)

    def weight_bytes(self):
        return sum(self.n_active * pw.nbytes() // pw.E for pw in self.layer.projs)

    def flops(self):
        return sum(2.0 * self.T * self.layer.cfg.k * pw.N * pw.K for pw in self.layer.projs)


class DequantSlot(StepSlot):
    """The same step (route, both projections on the same inputs, combine)
    through the dequantize-then-matmul path the pages compare against: the
    routed experts of each projection are decoded to bf16 in HBM
    (gnf4_dequant_experts_bf16), then multiplied with torch's library GEMMs
    (hipBLASLt / rocBLAS): one batched product at T = 1, one 2-D product per
    active expert otherwise (torch has no grouped GEMM)."""

    def __init__(self, torch, gnf4, cfg, layer, T, seed, wbuf):
        super().__init__(torch, gnf4, cfg, layer, T, seed)
        k = cfg.k
        ids = self.ids.cpu().numpy()
        self.wbuf = wbuf                       # bf16 decode buffers, one per projection
        self.counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
        self.segs = []                          # (slot, first routed row, rows)
        off = 0
        for e in range(cfg.E):
            c = int(self.counts[e])
            if c:
                self.segs.append((len(self.segs), off, c))
            off += c
        self.max_slots = min(cfg.E, T * k)
        perm = np.argsort(ids.reshape(-1), kind="stable")
        self.src = torch.from_numpy((perm // k).astype(np.int64)).cuda()
        self.Yb = [torch.empty((T * k, p.N), dtype=torch.bfloat16, device="cuda") for p in cfg.projs]

    def run(self, gnf4):
        import torch
        cfg, T, k = self.layer.cfg, self.T, self.layer.cfg.k
        r = gnf4.route(self.ids, cfg.E, out=self.r)
        ins = [self.X, self.Xd if len(cfg.projs) > 1 else None]
        for pi, pw in enumerate(self.layer.projs):
            W = gnf4.dequant_experts_bf16(pw, r["active"], r["n_active"], self.max_slots,
                                          self.wbuf[pi]).view(torch.bfloat16)
            Xb = ins[pi].view(torch.bfloat16)
            if T == 1:
                # slot s holds routed row s (distinct ids); a gathered input is the token row
                xs = Xb.expand(self.max_slots, -1) if pi == 0 else Xb
                torch.bmm(W[:self.max_slots], xs.contiguous().unsqueeze(2),
                          out=self.Yb[pi].view(self.max_slots, pw.N, 1))
            else:
                A = Xb.index_select(0, self.src) if pi == 0 else Xb
                for slot, p0, c in self.segs:
                    torch.mm(A[p0:p0 + c], W[slot].t(), out=self.Yb[pi][p0:p0 + c])
        last = len(cfg.projs) - 1
        self.Y[last].copy_(self.Yb[last])
        gnf4.combine(self.Y[last], r["inv"], self.tw, T, k, self.out)


class BackwardSlot(StepSlot):
    """One backward step through the frozen experts of the layer: route, then
    for each projection in reverse order the input gradient dA = dY . W' on
    the packed weights (gnf4_grouped_gemm_dx, one launch each), then the sum
    of each token's routed copies for the gathered first projection. Each
    projection's output gradient dY is a standalone bf16 N(0,1) matrix in
    routed order (the SwiGLU and combine backward steps between them need
    saved forward activations and are not part of the path)."""

    def __init__(self, torch, gnf4, cfg, layer, T, seed):
        import synth
        super().__init__(torch, gnf4, cfg, layer, T, seed)
        k = cfg.k
        self.dY = [torch.from_numpy(synth.grad_rows(cfg, T * k, p.N, seed, T + 7 * pi).view(np.int16)).cuda()
                   for pi, p in enumerate(cfg.projs)]
        self.dA = [torch.empty((T * k, p.K), dtype=torch.float32, device="cuda") for p in cfg.projs]
        self.ones = torch.ones((T, k), dtype=torch.float32, device="cuda")
        self.dX = torch.empty((T, cfg.projs[0].K), dtype=torch.float32, device="cuda")

    def run(self, gnf4):
        cfg, T, k = self.layer.cfg, self.T, self.layer.cfg.k
        r = gnf4.route(self.ids, cfg.E, out=self.r)
        for pi in reversed(range(len(self.layer.projs))):
            gnf4.grouped_gemm_dx(self.layer.projs[pi], self.dY[pi], r, T, k, self.dA[pi])
        gnf4.combine(self.dA[0], r["inv"], self.ones, T, k, self.dX)


class DequantBackwardSlot(BackwardSlot):
    """The same backward step through the dequantize-then-matmul path: the
    routed experts of each projection decoded to bf16 in HBM, then torch's
    library GEMMs dA = dY . W (torch.bmm at T = 1, one torch.mm per active
    expert otherwise), bf16 results widened to float32 for the token sum."""

    def __init__(self, torch, gnf4, cfg, layer, T, seed, wbuf):
        super().__init__(torch, gnf4, cfg, layer, T, seed)
        k = cfg.k
        ids = self.ids.cpu().numpy()
        self.wbuf = wbuf
        counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
        self.segs = []
        off = 0
        for e in range(cfg.E):
            c = int(counts[e])
            if c:
                self.segs.append((len(self.segs), off, c))
            off += c
        self.max_slots = min(cfg.E, T * k)
        self.dAb = [torch.empty((T * k, p.K), dtype=torch.bfloat16, device="cuda") for p in cfg.projs]

    def run(self, gnf4):
        import torch
        cfg, T, k = self.layer.cfg, self.T, self.layer.cfg.k
        r = gnf4.route(self.ids, cfg.E, out=self.r)
        for pi in reversed(range(len(self.layer.projs))):
            pw = self.layer.projs[pi]
            W = gnf4.dequant_experts_bf16(pw, r["active"], r["n_active"], self.max_slots,
                                          self.wbuf[pi]).view(torch.bfloat16)
            dYb = self.dY[pi].view(torch.bfloat16)
            if T == 1:
                torch.bmm(dYb.view(self.max_slots, 1, pw.N), W[:self.max_slots],
                          out=self.dAb[pi].view(self.max_slots, 1, pw.K))
            else:
                for slot, p0, c in self.segs:
                    torch.mm(dYb[p0:p0 + c], W[slot], out=self.dAb[pi][p0:p0 + c])
        self.dA[0].copy_(self.dAb[0])
        gnf4.combine(self.dA[0], r["inv"], self.ones, T, k, self.dX)


CHAIN_MAX = 256     # steps per captured graph


def gpu_lead(torch):
    """A short device-side spin on the current stream, enqueued just before a
    timed region: the host then submits the region's events and graph
    launches while the GPU is still busy, so the region starts with its
    work already queued and holds no host submission gap."""
    torch.cuda._sleep(2_000_000)


def time_steps(torch, gnf4, slots, steps, warmup):
    """Time exactly `steps` consecutive steps, step i on slot i % len(slots).

    After `warmup` untimed eager steps, the steps are captured as graphs of
    at most CHAIN_MAX consecutive steps (one graph of L = min(steps,
    CHAIN_MAX) steps replayed steps // L times, then one of the remaining
    steps). That sequence is replayed twice back to back on one stream, and
    HIP events recorded on that stream bracket the second pass: its graphs
    are queued while the first pass runs, so the timed steps hold no host
    submission latency (the first pass is more untimed warmup). The whole is
    bracketed by device synchronizations. Returns (GPU seconds per step from
    the events, mean packed bytes of the experts a step routes to, mean
    flops)."""
    G = len(slots)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(max(warmup, 1)):              # also warms the launch path for capture
            slots[i % G].run(gnf4)
    torch.cuda.synchronize()
    L = min(steps, CHAIN_MAX)
    graphs = []
    for n, reps in ((L, steps // L), (steps % L, 1)):
        if n == 0 or reps == 0:
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                slots[i % G].run(gnf4)
        graphs.append((g, reps))
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        gpu_lead(torch)
        for timed in (False, True):
            if timed:
                a.record(stream)
            for g, reps in graphs:
                for _ in range(reps):
                    g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    dt = a.elapsed_time(b) * 1e-3 / steps
    # step i of the timed run is slot (i mod L) mod G: every graph starts at slot 0
    idx = [(i % L) % G for i in range(steps)]
    per = np.mean([slots[j].weight_bytes() for j in idx])
    fl = np.mean([slots[j].flops() for j in idx])
    del graphs
    return dt, per, fl


def time_steps_eager(torch, gnf4, slots, steps, warmup):
    """Time `steps` consecutive steps launched one call at a time from the host
    (no graph), step i on slot i % len(slots), between HIP events on the
    launch stream: the time per step includes each launch's host submission
    cost wherever the GPU waits for it."""
    G = len(slots)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(max(warmup, 1)):
            slots[i % G].run(gnf4)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        a.record(stream)
        for i in range(steps):
            slots[i % G].run(gnf4)
        b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / steps


def time_read_probe(torch, gnf4, nbytes, launches=64):
    """Achievable HBM read rate for `nbytes` read once: gnf4_read_probe over
    rotating buffers that together exceed 3x the Infinity Cache, `launches`
    back-to-back launches in one graph bracketed by HIP events, the median
    per-launch time over the replays; the best of a few grid sizes. Returns
    (GB/s, us per launch, workgroups)."""
    n = -(-int(nbytes) // 16) * 16
    copies = int(max(4, np.ceil(3 * MALL_BYTES / n)))
    bufs = [torch.ones(n // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    best = None
    for wg in (0, 512, 1024, 2048, 4096):
        with torch.cuda.stream(stream):
            for i in range(copies):
                gnf4.read_probe(bufs[i], n, wg, sink)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(launches):
                gnf4.read_probe(bufs[i % copies], n, wg, sink)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(5)]
        with torch.cuda.stream(stream):
            g.replay()
            gpu_lead(torch)
            for a, b in evs:
                a.record(stream)
                g.replay()
                b.record(stream)
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3 / launches
        if best is None or us < best[1]:
            best = (n / (us * 1e-6) / 1e9, us, wg)
        del g
    del bufs
    torch.cuda.empty_cache()
    return best


def gate_up_launch(gnf4, sl):
    """The gate_up launch of the step: with the routing fused in at T = 1."""
    cfg = sl.layer.cfg
    if sl.T == 1:
        gnf4.route_grouped_gemm(sl.ids, sl.layer.projs[0], sl.X, out=sl.r, Y=sl.Y[0])
    else:
        gnf4.grouped_gemm(sl.layer.projs[0], sl.X, 1, sl.r, sl.T, cfg.k, sl.Y[0])


def down_launch(gnf4, sl):
    """The down launch of the step (T = 1: the GEMV with the combine fused;
    otherwise the GEMM and then the combine kernel)."""
    cfg = sl.layer.cfg
    gnf4.grouped_gemm_combine(sl.layer.projs[1], sl.Xd, sl.r, sl.tw, sl.T, cfg.k, sl.out, Y=sl.Y[1])


def gate_up_dx_launch(gnf4, sl):
    cfg = sl.layer.cfg
    gnf4.grouped_gemm_dx(sl.layer.projs[0], sl.dY[0], sl.r, sl.T, cfg.k, sl.dA[0])


def time_kernel(torch, gnf4, slots, steps, warmup, launch=gate_up_launch):
    """Mean duration of one launch of the gate_up GEMM (or of `launch`):
    `steps` launches rotating through the slots (route outputs computed
    beforehand) are captured in one graph, and HIP events recorded on the
    replay stream bracket its replays; the mean is elapsed time / launches,
    so host launch cost is excluded and the gaps between back-to-back
    launches are included."""
    for sl in slots:
        gnf4.route(sl.ids, sl.layer.cfg.E, out=sl.r)
    torch.cuda.synchronize()
    cfg = slots[0].layer.cfg
    G = max(len(slots), min(steps, 64))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(min(warmup, G)):
            launch(gnf4, slots[i % len(slots)])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(G):
            launch(gnf4, slots[i % len(slots)])
    torch.cuda.synchronize()
    reps = max(2, -(-steps // G))
    with torch.cuda.stream(stream):
        graph.replay()                                  # warm
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        gpu_lead(torch)
        for a, b in evs:
            a.record(stream)
            graph.replay()
            b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs]) / G
    byts = np.mean([slots[i % len(slots)].n_active * slots[i % len(slots)].layer.projs[0].nbytes()
                    // cfg.E for i in range(G)])
    fl = np.mean([2.0 * slots[i % len(slots)].T * cfg.k * slots[i % len(slots)].layer.projs[0].N
                  * slots[i % len(slots)].layer.projs[0].K for i in range(G)])
    del graph
    return float(np.median(ms)), float(byts), float(fl), G


def dx_kernel_name(cfg, T):
    """The HIP kernel gnf4_grouped_gemm_dx runs for this workload (the library
    picks it from T*k and the mean rows per active expert)."""
    rows = T * cfg.k
    experts = min(cfg.E, rows)
    mean = -(-rows // experts) if experts else 0
    return "gemv_dx_kernel" if rows <= 64 and mean <= 4 else "mfma_dx_kernel"


def gemm_kernel_name(cfg, T):
    """The HIP kernel gnf4_grouped_gemm runs for this workload's gate_up call
    (the library picks it from T*k and the format)."""
    if T * cfg.k <= 64:
        return "gemv1w_kernel" if T == 1 else "gemv_kernel"
    return "mfma16_kernel"


def profile_fields(path):
    """The `key: value` lines of a committed summary under profiles/ when the
    kernel source it names is unchanged since it was taken (else None)."""
    import hashlib
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    src = fields.get("kernel_source")
    if not src or "traffic_bytes_per_launch" not in fields:
        return None
    digest = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    return fields if digest == fields.get("source_sha256") else None


def profile_traffic(cfg_name, mode, kernel=None, proj="gate_up"):
    """HBM bytes per launch of the kernel that runs projection `proj` (the
    forward GEMM's, or the named kernel's) from the committed rocprofv3
    counter summary profiles/<kernel>-<proj>-<workload>-<mode>.txt, if the
    kernel's source is unchanged since the counters were taken (else None)."""
    import glob
    pattern = "%s-%s-%s-%s.txt" % (kernel or "*", proj, cfg_name, mode)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", pattern))):
        if kernel is None and "_dx_kernel" in os.path.basename(path):
            continue
        fields = profile_fields(path)
        if fields:
            return int(fields["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)
    return None, None


def cpu_baseline(cfg, T):
    """The float64 oracle on one decode step of this workload (route, both
    projections' dequant + matmul for the routed experts, combine)."""
    import synth
    from oracle import combine, grouped_gemm, mxfp4, nf4, routing
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threadpool_info = None
    cores = len(os.sched_getaffinity(0))
    ids, tw = synth.routing_inputs(cfg, T, seed=12345)
    active = sorted(set(int(v) for v in ids.reshape(-1)))
    packs = []
    for proj in cfg.projs:
        nb = proj.K // (32 if cfg.fmt == "mxfp4" else 64)
        codes = np.zeros((cfg.E, proj.N, proj.K // 2), dtype=np.uint8)
        scales = np.zeros((cfg.E, proj.N, nb), dtype=np.uint8 if cfg.fmt == "mxfp4" else np.float32)
        scales2 = None
        for e in active:
            W = synth.expert_weight(cfg, proj, e)
            codes[e], scales[e] = (mxfp4.quantize if cfg.fmt == "mxfp4" else nf4.quantize)(W)
        if cfg.fmt == "nf4_dq":
            q8, scales2 = nf4.double_quantize_absmax(scales.reshape(-1))
            scales = q8.reshape(cfg.E, proj.N, nb)
        packs.append((proj, codes, scales, scales2))
    X = synth.token_inputs(cfg, T)
    Xd = synth.down_inputs(cfg, T) if len(cfg.projs) > 1 else None
    limit = threadpool_limits(limits=cores) if threadpool_limits else None
    reps, t_total, byts = 0, 0.0, 0
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        r = routing.route(ids, cfg.E)
        Y = None
        for pi, (proj, codes, scales, scales2) in enumerate(packs):
            inp = X if pi == 0 else Xd
            Y = grouped_gemm.grouped_gemm(cfg.fmt, codes, scales, scales2, inp, 1 if pi == 0 else 0,
                                          r["offsets"], r["perm"], cfg.k, proj.N, proj.K)
        combine.combine(Y, r["inv"], tw, T, cfg.k)
        t_total += time.perf_counter() - t0
        reps += 1
        for proj, codes, scales, scales2 in packs:
            per = codes[0].nbytes + scales[0].nbytes
            byts += len(active) * per
        if time.perf_counter() - t_start > 12.0 or reps >= 400:
            break
    threads = cores
    if threadpool_info is not None:
        info = threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    if limit is not None:
        limit.unregister() if hasattr(limit, "unregister") else None
    return {"value": round(byts / t_total / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d full decode step(s) (T=%d, %d routed experts, both projections: dequant + "
                      "float64 matmul + combine), %.1f s" % (reps, T, len(active), t_total),
            "cpu_model": cpu_model()}


def packed_digest(layer):
    """sha256 of the layer's packed bytes (every projection's codes, scales and
    second-level scales, in order), read back from the device."""
    import hashlib
    h = hashlib.sha256()
    for pw in layer.projs:
        for t in (pw.codes, pw.scales, pw.scales2):
            if t is not None:
                h.update(t.contiguous().cpu().numpy().tobytes())
    return h.hexdigest()


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class StreamSlot:
    """One decode step of the layer streamed from host RAM: the residency
    decision, the fill of the missing experts into both projections' caches,
    then the step on the slot ids (route fused into the first projection,
    the second with the combine fused)."""

    def __init__(self, torch, gnf4, cfg, host, cache, state, S, ids, tw, X, Xd):
        k = cfg.k
        self.cfg, self.host, self.cache, self.state, self.S = cfg, host, cache, state, S
        self.ids = torch.from_numpy(np.ascontiguousarray(ids.reshape(1, k))).cuda()
        self.tw = torch.from_numpy(np.ascontiguousarray(tw.reshape(1, k))).cuda()
        self.X, self.Xd = X, Xd
        self.slot_ids = torch.empty((1, k), dtype=torch.int32, device="cuda")
        self.max_copies = min(k, cfg.E, S)
        self.copies = torch.zeros((1 + 2 * self.max_copies,), dtype=torch.int32, device="cuda")
        self.r = gnf4.route_buffers(1, k, S)
        self.Y = [torch.empty((k, pw.N), dtype=torch.float32, device="cuda") for pw in cache]
        self.out = torch.empty((1, cache[-1].N), dtype=torch.float32, device="cuda")

    def run(self, gnf4, resident=None):
        k = self.cfg.k
        if resident is not None:                 # the same step on the HBM-resident layer
            r, _ = gnf4.route_grouped_gemm(self.ids, resident[0], self.X, out=self.rr, Y=self.Y[0])
            gnf4.grouped_gemm_combine(resident[1], self.Xd, r, self.tw, 1, k, self.out, Y=self.Y[1])
            return
        gnf4.expert_cache_stage(self.ids, self.cfg.E, self.S, self.state, self.slot_ids, self.copies)
        for h, c in zip(self.host, self.cache):
            gnf4.expert_cache_fill(h, c, self.copies, self.max_copies)
        r, _ = gnf4.route_grouped_gemm(self.slot_ids, self.cache[0], self.X, out=self.r, Y=self.Y[0])
        gnf4.grouped_gemm_combine(self.cache[1], self.Xd, r, self.tw, 1, k, self.out, Y=self.Y[1])


def streaming(torch, gnf4, cfg, base, steps):
    """Decode steps (T = 1) of the layer with its packed experts in pinned host
    memory and an HBM cache of S = max(k, E/4) expert slots per projection,
    over a sequence of tokens routed by the workload's router. Returns the
    step time, the bytes streamed per step, the hit rate, the link ceilings
    (the fill kernel on all-miss copies; a pinned host-to-device copy) and
    the same steps on the HBM-resident layer."""
    import synth
    E, k = cfg.E, cfg.k
    S = max(k, E // 4)
    host = []
    for pw in base.projs:
        host.append(type(pw)(pw.format, pw.E, pw.N, pw.K, pw.codes.cpu().pin_memory(),
                             pw.scales.cpu().pin_memory(),
                             pw.scales2.cpu().pin_memory() if pw.scales2 is not None else None))
    cache = [gnf4.empty_packed(cfg.fmt, S, pw.N, pw.K) for pw in base.projs]
    state = gnf4.expert_cache_state(E, S)
    n = max(16, steps)
    ids, tw = synth.routing_inputs(cfg, n, seed=700)
    X = torch.from_numpy(synth.token_inputs(cfg, n, seed=700).view(np.int16)).cuda()
    Xd = torch.from_numpy(synth.activations(cfg, k, cfg.inter, synth.T_X_DOWN, 700, 1)
                          .view(np.int16)).cuda()
    slots = [StreamSlot(torch, gnf4, cfg, host, cache, state, S, ids[t], tw[t], X[t:t + 1], Xd)
             for t in range(n)]
    chain = torch.cuda.CUDAGraph()
    for sl in slots[:2]:
        sl.run(gnf4)                             # warm the launch path outside capture
    torch.cuda.synchronize()
    with torch.cuda.graph(chain):
        for sl in slots:
            sl.run(gnf4)
    torch.cuda.synchronize()
    chain.replay()                               # one pass to reach a steady cache
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    chain.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / n
    misses = np.array([int(sl.copies[0].item()) for sl in slots])
    per_expert = sum(pw.nbytes() // pw.E for pw in base.projs)
    n_need = np.array([np.unique(ids[t]).size for t in range(n)])
    streamed = float(misses.mean()) * per_expert

    # the same steps with the layer resident in HBM
    for sl in slots:
        sl.rr = gnf4.route_buffers(1, k, E)
    res = torch.cuda.CUDAGraph()
    with torch.cuda.graph(res):
        for sl in slots:
            sl.run(gnf4, resident=base.projs)
    torch.cuda.synchronize()
    res.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res.replay()
    torch.cuda.synchronize()
    dt_res = (time.perf_counter() - t0) / n

    # link ceilings for k experts' bytes: the fill kernel with every copy a
    # miss, and a pinned host-to-device copy of the same bytes
    m = min(k, S)
    cp = torch.tensor([m] + [v for i in range(m) for v in (i, i)], dtype=torch.int32, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for h, c in zip(host, cache):
        gnf4.expert_cache_fill(h, c, cp, m)
    torch.cuda.synchronize()
    reps = 5
    a.record()
    for _ in range(reps):
        for h, c in zip(host, cache):
            gnf4.expert_cache_fill(h, c, cp, m)
    b.record()
    torch.cuda.synchronize()
    fill_gbs = reps * m * per_expert / (a.elapsed_time(b) * 1e-3) / 1e9
    src = torch.empty((m * per_expert,), dtype=torch.uint8).pin_memory()
    dst = torch.empty((m * per_expert,), dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    copy_gbs = reps * m * per_expert / (a.elapsed_time(b) * 1e-3) / 1e9
    del slots, chain, res, cache, host, src, dst
    torch.cuda.empty_cache()
    return dict(S=S, n=n, dt=dt, dt_res=dt_res, streamed=streamed, per_expert=per_expert,
                misses=float(misses.mean()), needed=float(n_need.mean()), fill_gbs=fill_gbs,
                copy_gbs=copy_gbs)


def main():
    args = parse()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.kernel_only:
        kernel_only(args)
        return
    import torch

    import synth
    from bit_mixture_experts_topk_amd import gnf4
    gnf4.lib()
    cfg = synth.CONFIGS[args.config]
    torch.cuda.set_device(0)
    base = Layer(torch, gnf4, cfg)
    layer_bytes = base.nbytes()

    result = {"metric": "packed-weight GB/s (% of HBM peak) at bs=1; prefill TFLOP/s (% MFMA peak)",
              "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic"}
    T_dec = min(cfg.Ts)
    T_pre = max(cfg.Ts)
    decode_ok = T_dec * cfg.k <= 64 and args.only in (None, "decode")
    prefill_ok = T_pre * cfg.k > 64 and args.only in (None, "prefill")

    out = {}
    if decode_ok:
        # enough weight copies that a copy is reused only after > 2x MALL of other traffic
        step_bytes = layer_bytes * min(1.0, T_dec * cfg.k / cfg.E)
        copies = int(min(32, max(4, np.ceil(3 * MALL_BYTES / max(step_bytes, 1)))))
        layers = [base] + [base.clone(torch) for _ in range(copies - 1)]
        slots = [StepSlot(torch, gnf4, cfg, layers[i % copies], T_dec, seed=100 + i)
                 for i in range(max(copies, 16))]
        dt, byts, _ = time_steps(torch, gnf4, slots, args.steps, args.warmup)
        kms, kbytes, _, glaunch = time_kernel(torch, gnf4, slots, args.steps, args.warmup)
        out["decode"] = dict(T=T_dec, ms_per_step=dt * 1e3, gbs=byts / dt / 1e9,
                             kernel_us=kms * 1e3, kernel_bytes=kbytes, copies=copies,
                             graph_launches=glaunch)
        if len(cfg.projs) > 1:
            dms, _, _, _ = time_kernel(torch, gnf4, slots, args.steps, args.warmup, down_launch)
            dbytes = np.mean([sl.n_active * sl.layer.projs[1].nbytes() // cfg.E for sl in slots])
            out["decode"]["down"] = (dms * 1e3, dbytes)
        del slots, layers
        torch.cuda.empty_cache()
        out["decode"]["read"] = time_read_probe(torch, gnf4, kbytes)
    if prefill_ok:
        copies = int(min(8, max(2, np.ceil(3 * MALL_BYTES / max(layer_bytes, 1)))))
        layers = [base] + [base.clone(torch) for _ in range(copies - 1)]
        slots = [StepSlot(torch, gnf4, cfg, layers[i % copies], T_pre, seed=200 + i)
                 for i in range(copies)]
        steps = max(10, args.steps // 10)
        dt, byts, fl = time_steps(torch, gnf4, slots, steps, max(2, args.warmup // 5))
        kms, kbytes, kfl, _ = time_kernel(torch, gnf4, slots, steps, max(2, args.warmup // 5))
        out["prefill"] = dict(T=T_pre, ms_per_step=dt * 1e3, tflops=fl / dt / 1e12, steps=steps,
                              kernel_us=kms * 1e3, kernel_flops=kfl, copies=copies)
        if len(cfg.projs) > 1:
            dms, _, _, _ = time_kernel(torch, gnf4, slots, steps, max(2, args.warmup // 5), down_launch)
            dn = cfg.projs[1]
            dfl = np.mean([2.0 * sl.T * cfg.k * dn.N * dn.K for sl in slots])
            out["prefill"]["down"] = (dms * 1e3, dfl)
        del slots, layers
        torch.cuda.empty_cache()

    if len(cfg.projs) > 1 and args.only is None:
        # the whole FFN layer (router top-k, gate_up, SwiGLU, down, combine)
        ffn = {}
        for T, tag in ((T_dec, "decode"), (T_pre, "prefill")):
            if (tag == "decode") != (T * cfg.k <= 64):
                continue
            step_bytes = layer_bytes * min(1.0, T * cfg.k / cfg.E)
            copies = int(min(32 if tag == "decode" else 8,
                             max(2, np.ceil(3 * MALL_BYTES / max(step_bytes, 1)))))
            layers = [base] + [base.clone(torch) for _ in range(copies - 1)]
            nsl = max(copies, 16) if tag == "decode" else copies
            slots = [StepSlot(torch, gnf4, cfg, layers[i % copies], T, seed=300 + i, ffn=True)
                     for i in range(nsl)]
            steps = args.steps if tag == "decode" else max(10, args.steps // 10)
            dt, byts, fl = time_steps(torch, gnf4, slots, steps, max(2, args.warmup // 5))
            ffn[tag] = (T, dt, byts, fl)
            del slots, layers
            torch.cuda.empty_cache()
        out["ffn"] = ffn

    if args.only is None and not args.no_dequant_path:
        # the dequantize-then-matmul comparison path, same steps and inputs
        dq = {}
        for T, tag in ((T_dec, "decode"), (T_pre, "prefill")):
            if not ((tag == "decode" and decode_ok) or (tag == "prefill" and prefill_ok)):
                continue
            step_bytes = layer_bytes * min(1.0, T * cfg.k / cfg.E)
            copies = int(min(32 if tag == "decode" else 4,
                             max(2, np.ceil(3 * MALL_BYTES / max(step_bytes, 1)))))
            layers = [base] + [base.clone(torch) for _ in range(copies - 1)]
            ms = min(cfg.E, T * cfg.k)
            wbuf = [torch.empty((ms, pw.N, pw.K), dtype=torch.int16, device="cuda") for pw in base.projs]
            nsl = max(copies, 16) if tag == "decode" else copies
            slots = [DequantSlot(torch, gnf4, cfg, layers[i % copies], T, 400 + i, wbuf)
                     for i in range(nsl)]
            steps = args.steps if tag == "decode" else max(10, args.steps // 10)
            dt, byts, fl = time_steps(torch, gnf4, slots, steps, max(2, args.warmup // 5))
            dt_eager = time_steps_eager(torch, gnf4, slots, steps, max(2, args.warmup // 5))
            del slots
            fslots = [StepSlot(torch, gnf4, cfg, layers[i % copies], T, 400 + i) for i in range(nsl)]
            fused_eager = time_steps_eager(torch, gnf4, fslots, steps, max(2, args.warmup // 5))
            dq[tag] = (T, dt, dt_eager, fused_eager)
            del fslots, layers, wbuf
            torch.cuda.empty_cache()
        out["dequant"] = dq

    if args.only in (None, "backward"):
        # backward through the frozen experts: input gradients of every projection
        bw = {}
        for T, tag in ((T_dec, "decode"), (T_pre, "prefill")):
            if tag == "decode" and T * cfg.k > 64:
                continue
            step_bytes = layer_bytes * min(1.0, T * cfg.k / cfg.E)
            copies = int(min(32 if tag == "decode" else 8,
                             max(2, np.ceil(3 * MALL_BYTES / max(step_bytes, 1)))))
            layers = [base] + [base.clone(torch) for _ in range(copies - 1)]
            nsl = max(copies, 16) if tag == "decode" else copies
            slots = [BackwardSlot(torch, gnf4, cfg, layers[i % copies], T, seed=500 + i)
                     for i in range(nsl)]
            steps = args.steps if tag == "decode" else max(10, args.steps // 10)
            wu = max(2, args.warmup // 5)
            dt, byts, fl = time_steps(torch, gnf4, slots, steps, wu)
            kms, kbytes, kfl, _ = time_kernel(torch, gnf4, slots, steps, wu, gate_up_dx_launch)
            entry = dict(T=T, dt=dt, byts=byts, fl=fl, kms=kms, kbytes=kbytes, kfl=kfl)
            del slots
            if not args.no_dequant_path:
                ms = min(cfg.E, T * cfg.k)
                wbuf = [torch.empty((ms, pw.N, pw.K), dtype=torch.int16, device="cuda") for pw in base.projs]
                nd = min(nsl, 16 if tag == "decode" else 4)
                dslots = [DequantBackwardSlot(torch, gnf4, cfg, layers[i % copies], T, 600 + i, wbuf)
                          for i in range(nd)]
                entry["dq_dt"] = time_steps(torch, gnf4, dslots, steps, wu)[0]
                del dslots, wbuf
            bw[tag] = entry
            del layers
            torch.cuda.empty_cache()
        out["backward"] = bw

    if len(cfg.projs) > 1 and args.only in (None, "streaming") and T_dec * cfg.k <= 64:
        out["streaming"] = streaming(torch, gnf4, cfg, base, min(args.steps, 256))

    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    wl = {"workload": "%s-shaped MoE FFN layer: E=%d top-%d, d=%d, I=%d, %s (block %d); "
                      "decode T=%s, prefill T=%s" % (cfg.name, cfg.E, cfg.k, cfg.d, cfg.inter,
                                                     cfg.fmt.upper(), 32 if cfg.fmt == "mxfp4" else 64,
                                                     T_dec if decode_ok else "-",
                                                     T_pre if prefill_ok else "-"),
          "global_batch": T_dec if decode_ok else T_pre, "layer_packed_MB": round(layer_bytes / 1e6, 2),
          "packed_sha256": packed_digest(base), "parallelism": "single GPU"}
    result["config"] = wl
    if "decode" in out:
        d = out["decode"]
        result["value"] = round(d["gbs"], 2)
        result["ms_per_step"] = round(d["ms_per_step"], 5)
        ach = d["kernel_bytes"] / (d["kernel_us"] * 1e-6) / 1e9
        traffic, tsrc = profile_traffic(cfg.name, "decode")
        rd_gbs, rd_us, rd_wg = d["read"]
        result["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                              "traffic_unit": "HBM bytes/launch", "traffic_source": tsrc,
                              "kernel": "%s (gate_up, T=%d)" % (gemm_kernel_name(cfg, d["T"]), d["T"]),
                              "kernel_us": round(d["kernel_us"], 3),
                              "launches_per_graph": d["graph_launches"],
                              "bytes_per_launch": int(d["kernel_bytes"]),
                              "achievable_read_GBps": round(rd_gbs, 1),
                              "achievable_read_us": round(rd_us, 3),
                              "frac_of_achievable_read": round(ach / rd_gbs, 4),
                              "achievable_read_kernel": "read_probe_kernel (gnf4_read_probe, %s "
                                                        "workgroups, the same bytes per launch)"
                                                        % (rd_wg or "8/CU")}
        result["decode"] = {"step_us": round(d["ms_per_step"] * 1e3, 3),
                            "pct_hbm_peak_step": round(100 * d["gbs"] / HBM_PEAK_GBS, 2),
                            "weight_copies": d["copies"]}
        if "down" in d:
            dus, dbytes = d["down"]
            dtr, dsrc = profile_traffic(cfg.name, "decode", "gemv1c_kernel", "down")
            result["decode"]["down_kernel"] = {
                "kernel": "gemv1c_kernel (down GEMV + combine, T=%d)" % d["T"],
                "kernel_us": round(dus, 3), "bytes_per_launch": int(dbytes),
                "GBps": round(dbytes / (dus * 1e-6) / 1e9, 1),
                "frac_hbm_peak": round(dbytes / (dus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "traffic": dtr, "traffic_source": dsrc}
    if "prefill" in out:
        p = out["prefill"]
        kt = p["kernel_flops"] / (p["kernel_us"] * 1e-6) / 1e12
        ptraffic, ptsrc = profile_traffic(cfg.name, "prefill")
        result["prefill"] = {"T": p["T"], "steps": p["steps"], "step_ms": round(p["ms_per_step"], 4),
                             "tflops": round(p["tflops"], 2),
                             "pct_mfma_peak_step": round(100 * p["tflops"] / BF16_PEAK_TFLOPS, 2),
                             "roofline": {"bound": "mfma", "achieved": round(kt, 2),
                                          "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                          "frac": round(kt / BF16_PEAK_TFLOPS, 4), "traffic": ptraffic,
                                          "traffic_unit": "HBM bytes/launch", "traffic_source": ptsrc,
                                          "kernel": "%s (gate_up, T=%d)" % (gemm_kernel_name(cfg, p["T"]), p["T"]),
                                          "kernel_us": round(p["kernel_us"], 2)}}
        if "down" in p:
            dus, dfl = p["down"]
            dtr, dsrc = profile_traffic(cfg.name, "prefill", "mfma16_kernel", "down")
            result["prefill"]["down_kernel"] = {
                "kernel": "mfma16_kernel + combine_kernel (down GEMM, then the combine, T=%d)" % p["T"],
                "us": round(dus, 2), "gemm_flops": dfl,
                "tflops": round(dfl / (dus * 1e-6) / 1e12, 2),
                "frac_mfma_peak": round(dfl / (dus * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "gemm_traffic": dtr, "traffic_source": dsrc}
        if "decode" not in out:
            result["value"] = round(p["tflops"], 3)
            result["unit"] = "TFLOP/s"
            result["ms_per_step"] = round(p["ms_per_step"], 5)
            result["roofline"] = result["prefill"]["roofline"]
    if out.get("ffn"):
        f = {}
        if "decode" in out["ffn"]:
            T, dt, byts, _ = out["ffn"]["decode"]
            f["decode"] = {"T": T, "step_us": round(dt * 1e6, 3), "packed_GBps": round(byts / dt / 1e9, 2),
                           "pct_hbm_peak": round(100 * byts / dt / 1e9 / HBM_PEAK_GBS, 2)}
        if "prefill" in out["ffn"]:
            T, dt, _, fl = out["ffn"]["prefill"]
            f["prefill"] = {"T": T, "step_ms": round(dt * 1e3, 4), "tflops": round(fl / dt / 1e12, 2),
                            "pct_mfma_peak": round(100 * fl / dt / 1e12 / BF16_PEAK_TFLOPS, 2)}
        f["steps"] = ("router top-k + softmax + route + gate_up GEMM with the SwiGLU epilogue "
                      "(bf16 H) (gnf4_route_logits_grouped_gemm), down GEMM on H + combine "
                      "(gnf4_grouped_gemm_combine): two launches at T = 1")
        f["parity_bars"] = ("each GEMM call: max|err| <= 1e-2*rms and rel. Frobenius <= 2e-3 of the "
                            "fp64 oracle; SwiGLU H: <= 2^-6*max|H|, Frobenius <= 6e-3; layer output "
                            "(gate_up error through SwiGLU + H rounding + down error): max|err| <= "
                            "3e-2*rms, Frobenius <= 6e-3 (tests/tolerance.py; tests/test_gpu_fullsize.py "
                            "checks every element of this step at T = 1)")
        result["ffn_layer"] = f
    if out.get("dequant"):
        dqr = {}
        for tag, (T, dt, dt_eager, fused_eager) in out["dequant"].items():
            fused = out[tag]["ms_per_step"] * 1e-3 if tag in out else None
            dqr[tag] = {"T": T, "step_us": round(dt * 1e6, 2),
                        "fused_speedup": round(dt / fused, 3) if fused else None,
                        "ungraphed_step_us": round(dt_eager * 1e6, 2),
                        "fused_ungraphed_step_us": round(fused_eager * 1e6, 2),
                        "fused_ungraphed_vs_graphed_dequant": round(dt / fused_eager, 3)}
        dqr["steps"] = ("route, bf16 dequant of the routed experts of each projection "
                        "(gnf4_dequant_experts_bf16), torch.bmm (T = 1) or one torch.mm per "
                        "active expert (library GEMMs), combine; same inputs as the fused step; "
                        "step_us replays the steps as graphs, ungraphed_step_us launches them "
                        "from the host one call at a time (both event-timed on the GPU), and "
                        "fused_ungraphed_vs_graphed_dequant is the graphed dequant step over "
                        "the host-launched fused step")
        result["dequant_path"] = dqr
    if out.get("backward"):
        b = {}
        for tag, en in out["backward"].items():
            item = {"T": en["T"], "step_us": round(en["dt"] * 1e6, 2)}
            kt = en["kfl"] / (en["kms"] * 1e-3) / 1e12
            kg = en["kbytes"] / (en["kms"] * 1e-3) / 1e9
            kname = dx_kernel_name(cfg, en["T"])
            name = "%s (gate_up, T=%d)" % (kname, en["T"])
            if tag == "decode":
                item["packed_GBps"] = round(en["byts"] / en["dt"] / 1e9, 2)
                tr, tsrc = profile_traffic(cfg.name, "decode", kname)
                item["roofline"] = {"bound": "hbm", "achieved": round(kg, 1), "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": round(kg / HBM_PEAK_GBS, 4),
                                    "traffic": tr, "traffic_unit": "HBM bytes/launch",
                                    "traffic_source": tsrc, "kernel": name,
                                    "kernel_us": round(en["kms"] * 1e3, 3),
                                    "bytes_per_launch": int(en["kbytes"])}
            else:
                item["tflops"] = round(en["fl"] / en["dt"] / 1e12, 2)
                tr, tsrc = profile_traffic(cfg.name, "prefill", kname)
                item["roofline"] = {"bound": "mfma", "achieved": round(kt, 2), "peak": BF16_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(kt / BF16_PEAK_TFLOPS, 4),
                                    "traffic": tr, "traffic_unit": "HBM bytes/launch",
                                    "traffic_source": tsrc, "kernel": name,
                                    "kernel_us": round(en["kms"] * 1e3, 2)}
            if "dq_dt" in en:
                item["dequant_path_step_us"] = round(en["dq_dt"] * 1e6, 2)
                item["fused_speedup"] = round(en["dq_dt"] / en["dt"], 3)
            b[tag] = item
        b["steps"] = ("route, gnf4_grouped_gemm_dx on down then gate_up (one launch each, packed "
                      "weights), sum of each token's routed copies (gnf4_combine, unit weights); "
                      "dequant_path: bf16 decode of the routed experts + torch.bmm / torch.mm")
        result["backward"] = b
    if out.get("streaming"):
        st = out["streaming"]
        link = st["fill_gbs"]
        model = st["streamed"] / (link * 1e9) + st["dt_res"]
        result["streaming"] = {
            "T": 1, "cache_slots": st["S"], "steps": st["n"],
            "step_us": round(st["dt"] * 1e6, 2), "resident_step_us": round(st["dt_res"] * 1e6, 2),
            "experts_needed_per_step": round(st["needed"], 3),
            "experts_streamed_per_step": round(st["misses"], 3),
            "hit_rate": round(1 - st["misses"] / st["needed"], 4),
            "streamed_MB_per_step": round(st["streamed"] / 1e6, 3),
            "fill_link_GBps": round(st["fill_gbs"], 2), "h2d_copy_GBps": round(st["copy_gbs"], 2),
            "model_step_us": round(model * 1e6, 2),
            "step_over_model": round(st["dt"] / model, 3),
            "steps_desc": ("gnf4_expert_cache_stage, gnf4_expert_cache_fill of both projections "
                           "from pinned host memory, then the decode step on the slot ids; model = "
                           "streamed bytes / fill_link_GBps + resident_step_us"),
        }
    if not args.no_cpu and decode_ok:
        result["cpu_baseline"] = cpu_baseline(cfg, T_dec)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
