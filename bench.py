"""Throughput of the Clebsch-Gordan tensor-product convolution on one MI355X.

Default: one step = forward + backward (gradients of x, phi, A and the positions) of the
channelwise convolution on the 1,024-atom perturbed-diamond graph (cutoff 5 A, ~91k directed
edges), 128x0e+128x1o+128x2e -> 128x(0e,1o,2e,3o), SH lmax 3, 8 radial functions, float32,
inputs resident in device memory.  Prints one JSON line:

  metric / value / unit      edges per second of the step (whole job, one GPU)
  kernels                    per kernel: launches and time per step (HIP events recorded around
                             every launch on its stream), algorithmic TFLOP/s where defined
  roofline                   the dominant kernel against its peak (vector ALU or MFMA)
  cpu_baseline               the float64 CPU oracle on a bounded receiver slice of the same
                             workload, timed on this host (a reported baseline, not a target)

``--workload N`` measures another of the five standard workloads with its own passes (1: both
forward schedules; 3: forward, float64; 4: fully connected streamed forward + backward; 5:
forward + backward + double backward); ``--copy-probe`` only runs a device copy of known size,
which calibrates the HBM byte counters of rocprofv3.

``--sweep degree|copies`` runs the scaling axes of the Sobek page's section 5.1 (fully connected
irrep profiles 128/64, 128/64/64, 128/64/64/64; ``--profile L`` picks one): per point one JSON
line with forward and backward time, edges/s, the library's workspace for each pass, the bytes
a materialised E x N_w weight tensor would take, and the peak device allocation of the point.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = 2
# Published MI355X vector peaks: fp32 157.3 TFLOP/s (counted with packed fp32 FMA, two per lane
# per cycle), fp64 78.6.  The kernels are built without packed fp32 instructions, so the vector
# FMA rate they can reach is 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz = 78.6 TFLOP/s in
# either precision; both fractions are reported, and the measured FMA rate of a plain probe kernel
# beside them.  Dense MFMA: fp32 157.3, fp64 78.6.  HBM 8 TB/s.
PEAK_ALU_UNPACKED_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
PEAK_ALU_PUBLISHED_TFLOPS = {"float32": 157.3, "float64": 78.6}
PEAK_MFMA_TFLOPS = {"float32": 157.3, "float64": 78.6}
PEAK_HBM_GBS = 8000.0
PREROLL_MS = 100.0          # untimed steps before the warm-up, so that the clocks have ramped
PROTOCOL_MIN_MS = 250.0     # sample time of the median protocol (Sobek section 5.1)
PROTOCOL_MIN_SAMPLES = 10

# Scratch budget per workload when --scratch-mib is not given: the library's default (256 MiB) for
# the small ones; the 16k-atom fully connected and the l <= 6 workloads are quoted with budgets that
# hold their receiver state (4 GiB) and coefficient rows (16 GiB) in one chunk (of 288 GB of HBM).
WORKLOAD_SCRATCH_MIB = {4: 4096, 5: 16384}
PASSES = {1: ("fwd", "fwds"), 2: ("fwd", "bwd"), 3: ("fwd",), 4: ("fwds", "bwd"), 5: ("fwd", "bwd", "dbl")}
PASS_NAMES = {"fwd": "forward (conventional)", "fwds": "forward (streamed)", "bwd": "backward",
              "dbl": "double backward"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "cgtp_bwd_recv__diamond1024_uvu_l3_fp32__hbm_counters.md")


def _blocks(irreps: str):
    out = []
    for tok in irreps.split("+"):
        m = re.fullmatch(r"(\d+)x(\d+)([eo])", tok.strip())
        out.append((int(m.group(1)), int(m.group(2))))
    return out


def _path_table(plan):
    rows = []
    for k in range(plan.info["n_paths"]):
        d = plan.path(k)
        idx, _ = plan.cg_table(k)
        rows.append(dict(d, gnz=len({(int(a), int(c)) for a, _, c in idx}),
                         p12=len({(int(a), int(b)) for a, b, _ in idx}), nnz=len(idx),
                         d1=2 * d["l1"] + 1, d2=2 * d["l2"] + 1, d3=2 * d["l3"] + 1))
    return rows


def kernel_fma(plan, spec, n_edges: int, n_nodes: int, passes, keep_state: bool = False):
    """Algorithmic FMA per step of each kernel, from the plan's path table.

    Per path with C channels (uvu), K radial functions, gnz (m1, m3) pairs, p12 (m1, m2) pairs, nnz
    CG terms and component counts d1, d2, d3, per edge:
      prep            nnz (G = sum c Y), once per pass that needs it
      fwd / bwd_src   C (K + gnz + min(d1, d3)): w = phi A, T = G x (or G^T mbar), w applied on the
                      smaller side
      fwd_streamed    C (gnz + K d3) per edge plus C K d3 per receiver (S, then S A)
      bwd_recv        the cheaper exact form: C (2 gnz + 3K + d3) + 2 nnz with T = G x, or, folding
                      R = sum c mbar once per receiver (C nnz), C (p12 + 2 d2 + 3K)
      prep2           2 nnz (G and its tangent)
      dfwd            C (3K + 3 gnz + 2 d3): w, wdot, T, Tdot, mdot
      drecv           C (7K + 5 gnz + 2 d3 + 2 d1) + 2 nnz: the tangents of h, A-bar, phi-bar and
                      Y-bar and the first-order Y-bar, as written in the method's equations
      dsrc            C (3K + 2 gnz + 2 d1)
    Fully connected (C_in, C_out per path):
      uvw_state       C_in (gnz + K d3) per edge, in every pass that forms S (the forward only
                      when the backward reads the state the forward kept)
      uvw_edge        C_in (gnz + 2 K d3 + nnz) per edge: T, phi-bar = sum Sbar T, Cbar = sum phi Sbar
                      and the Y-bar contraction
      uvw_zstate      C_out (gnz + K d1) per edge
      gemm_fwd<g>, gemm_sbar<g>, gemm_abar<g>: (N d3_g) x C_out x sum_{paths into g} K C_in
      gemm_xbar<b>    (N d1_b) x C_in x sum_{paths from b} K C_out
    The fully connected double backward (every direction given) runs the state kernel and the
    forward GEMMs four times (three terms of S-dot, and S for S A-dot), the A-bar GEMMs three
    times, the Sbar GEMMs twice, the edge kernel four times (three tangent passes and the
    first-order Y-bar), and the source state and x-bar GEMMs three times.
    Kernels without an entry (edge finalisation, reductions) are reported by time only.
    """
    K, E, N = plan.info["num_radial"], n_edges, n_nodes
    deg = E / max(N, 1)
    rows = _path_table(plan)
    f = {}

    def add(name, v):
        f[name] = f.get(name, 0.0) + v

    if spec["mode"] == "uvu":
        nnz = sum(r["nnz"] for r in rows)
        fwd = sum(r["n_weights"] * (K + r["gnz"] + min(r["d1"], r["d3"])) for r in rows) * E
        for ps in passes:
            if ps in ("fwd", "fwds") or (ps == "bwd" and not keep_state):
                add("cgtp_prep", nnz * E)
            if ps == "fwd":
                add("cgtp_fwd", fwd)
            if ps == "fwds":
                add("cgtp_fwd_streamed", sum(r["n_weights"] * (r["gnz"] + K * r["d3"]) * E
                                             + r["n_weights"] * K * r["d3"] * N for r in rows))
            if ps == "bwd":
                recv = 0.0
                for r in rows:
                    C = r["n_weights"]
                    plain = C * (2 * r["gnz"] + 3 * K + r["d3"]) + 2 * r["nnz"]
                    fold = C * (r["p12"] + 2 * r["d2"] + 3 * K) + C * r["nnz"] / deg
                    recv += min(plain, fold)
                add("cgtp_bwd_recv", recv * E)
                add("cgtp_bwd_src", fwd)
            if ps == "dbl":
                add("cgtp_prep2", 2 * nnz * E)
                add("cgtp_dfwd", sum(r["n_weights"] * (3 * K + 3 * r["gnz"] + 2 * r["d3"]) for r in rows) * E)
                add("cgtp_drecv", (sum(r["n_weights"] * (7 * K + 5 * r["gnz"] + 2 * r["d3"] + 2 * r["d1"])
                                       for r in rows) + 2 * nnz) * E)
                add("cgtp_dsrc", sum(r["n_weights"] * (3 * K + 2 * r["gnz"] + 2 * r["d1"]) for r in rows) * E)
        return f
    bi, bo = _blocks(spec["irreps_in"]), _blocks(spec["irreps_out"])
    state = sum(bi[r["i_in"]][0] * (r["gnz"] + K * r["d3"]) for r in rows) * E
    for ps in passes:
        if ps == "fwds" or (ps == "bwd" and not keep_state):
            add("cgtp_uvw_state", state)
        for g in sorted({r["i_out"] for r in rows}):
            depth = sum(K * bi[r["i_in"]][0] for r in rows if r["i_out"] == g)
            mac = N * (2 * bo[g][1] + 1) * bo[g][0] * depth
            if ps == "fwds":
                add(f"cgtp_gemm_fwd{g}", mac)
            if ps == "bwd":
                add(f"cgtp_gemm_sbar{g}", mac)
                add(f"cgtp_gemm_abar{g}", mac)
        # Launch multiplicities: (state, gemm_fwd, gemm_sbar, gemm_abar, edge, zstate, gemm_xbar).
        mult = {"fwds": (0, 1, 0, 0, 0, 0, 0), "bwd": (0, 0, 1, 1, 1, 1, 1), "dbl": (4, 4, 2, 3, 4, 3, 3)}.get(ps)
        if ps == "dbl":
            add("cgtp_uvw_state", 4 * state)
            for g in sorted({r["i_out"] for r in rows}):
                depth = sum(K * bi[r["i_in"]][0] for r in rows if r["i_out"] == g)
                mac = N * (2 * bo[g][1] + 1) * bo[g][0] * depth
                add(f"cgtp_gemm_fwd{g}", mult[1] * mac)
                add(f"cgtp_gemm_sbar{g}", mult[2] * mac)
                add(f"cgtp_gemm_abar{g}", mult[3] * mac)
        if ps in ("bwd", "dbl"):
            add("cgtp_uvw_edge", mult[4] * sum(bi[r["i_in"]][0] * (r["gnz"] + 2 * K * r["d3"] + r["nnz"])
                                               for r in rows) * E)
            add("cgtp_uvw_zstate", mult[5] * sum(bo[r["i_out"]][0] * (r["gnz"] + K * r["d1"]) for r in rows) * E)
            for b in sorted({r["i_in"] for r in rows}):
                depth = sum(K * bo[r["i_out"]][0] for r in rows if r["i_in"] == b)
                add(f"cgtp_gemm_xbar{b}", mult[6] * N * (2 * bi[b][1] + 1) * bi[b][0] * depth)
    return f


def generator_digest() -> str:
    """Hash of the kernel generator sources: HBM counters are valid for the code they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "clebsch_gordan_tensor_receiver_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith("codegen") or name in ("plan.cpp", "plan.hpp", "kernels.hpp", "runtime.cpp"):
            with open(os.path.join(csrc, name), "rb") as fh:
                h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if it was taken on the
    current kernel generator (else None)."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    dig = re.search(r"generator digest: `([0-9a-f]+)`", text)
    m = re.search(r"traffic bytes per launch of " + re.escape(kernel) + r": `([0-9.]+)`", text)
    if not dig or not m or dig.group(1) != generator_digest():
        return None
    return float(m.group(1))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--profile-steps", type=int, default=10)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=sorted(PASSES))
    ap.add_argument("--scratch-mib", type=int, default=0,
                    help="scratch budget of the plan in MiB (0: 4096 for workload 4, 16384 for workload 5, "
                         "else the library default of 256)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peak-probe", action="store_true",
                    help="skip the measured FMA and copy ceilings (cgtp_measure_peak)")
    ap.add_argument("--recompute-state", action="store_true",
                    help="let the backward recompute its state (fully connected: the receiver state; channelwise: "
                         "the per-edge coefficient rows) instead of reading the one the forward kept "
                         "(cgtp_conv_forward_keep_state)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of known size (calibrates the HBM byte counters)")
    ap.add_argument("--sweep", choices=("degree", "copies", "channels", "lmax", "skew"),
                    help="scaling axis of the fully connected profiles (one JSON line per point)")
    ap.add_argument("--profile", type=int, default=0, choices=(0, 1, 2, 3),
                    help="irrep profile (L_max) of the sweep; 0: all three")
    ap.add_argument("--radial", action="store_true",
                    help="compute the radial basis in the kernels from |r| (Bessel + envelope; Gaussians for "
                         "workload 5) instead of reading phi")
    ap.add_argument("--order", type=int, default=2, choices=(0, 1, 2),
                    help="node dispatch order of the graph: 0 index, 1 by degree, 2 automatic (default)")
    ap.add_argument("--double", action="store_true",
                    help="add the double backward to the workload's passes (the l <= 6 workload has it already; "
                         "with workload 4 the fully connected double backward)")
    ap.add_argument("--triple", action="store_true",
                    help="measure the third-order derivative (LunaTP Algorithm 4) on the workload's graph and "
                         "irreps, edge operand = the harmonics of the edge vectors, all directions and cotangents "
                         "present, fp32/fp64 as the workload")
    ap.add_argument("--points", default="",
                    help="comma-separated sweep points (degrees or copy counts); default: the whole axis")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the convolution runs on a single MI355X)", file=sys.stderr)
        return 2

    import torch

    import clebsch_gordan_tensor_receiver_amd as cg
    from workloads import CONFIGS, make_workload, normal_tensor

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.copy_probe:
        return copy_probe(torch)
    if args.sweep:
        return sweep(torch, cg, args)
    cfg = args.workload
    passes = PASSES[cfg]
    if args.double and "dbl" not in passes:
        passes = passes + ("dbl",)
    spec = CONFIGS[cfg]
    w = make_workload(cfg)
    dtype = spec["dtype"]
    plan = cg.Plan(spec["irreps_in"], spec["irreps_sh"], spec["irreps_out"], spec["mode"], dtype, spec["K"])
    if args.scratch_mib <= 0:
        args.scratch_mib = WORKLOAD_SCRATCH_MIB.get(cfg, 256)
    plan.set_scratch_budget(args.scratch_mib << 20)
    if args.radial:
        plan.set_radial(2 if spec["radial"] == "gaussian" else 1, spec["rc"])
    graph = cg.Graph(w.n_nodes, w.recv, w.send, w.image)
    graph.set_order(args.order)
    perm = graph.perm
    info = plan.info
    K, E, N = spec["K"], graph.n_edges, w.n_nodes
    if args.triple:
        return triple_bench(torch, cg, args, cfg, spec, w, plan, graph)
    tdt = torch.float64 if dtype == "float64" else torch.float32
    dev = dict(dtype=tdt, device="cuda")
    rnd = (lambda a: a.astype(np.float32).astype(np.float64)) if dtype == "float32" else (lambda a: a)
    x_h = normal_tensor(cfg, 1, (N, info["c_in"]), dtype=dtype)
    A_h = normal_tensor(cfg, 2, (K, info["n_weights"]), std=1.0 / np.sqrt(K), dtype=dtype)
    g_h = normal_tensor(cfg, 3, (N, info["c_out"]), dtype=dtype)
    x = torch.tensor(x_h, **dev)
    A = torch.tensor(A_h, **dev)
    gout = torch.tensor(g_h, **dev)
    pos = torch.tensor(rnd(w.pos), **dev)
    shift = torch.tensor(rnd(w.shift[perm]), **dev).contiguous()
    phi = torch.tensor(rnd(w.phi[perm]), **dev).contiguous()
    conv = cg.Convolution(plan, graph)
    ops = {"fwd": cg.OP_FORWARD, "fwds": cg.OP_FORWARD, "bwd": cg.OP_BACKWARD, "dbl": cg.OP_DOUBLE_BACKWARD}
    plan.compile(tuple(sorted({ops[p] for p in passes})))
    graph.upload()

    out = torch.empty((N, info["c_out"]), **dev)
    grads = dict(x=torch.empty_like(x), pos=torch.empty_like(pos), edge_vec=torch.empty((E, 3), **dev),
                 phi=torch.empty_like(phi), A=torch.empty_like(A))
    ws = {p: conv.workspace(ops[p]) for p in passes}
    if "dbl" in passes:
        dirs = dict(v_x=torch.tensor(normal_tensor(cfg, 4, (N, info["c_in"]), dtype=dtype), **dev),
                    v_pos=torch.tensor(normal_tensor(cfg, 5, (N, 3), dtype=dtype), **dev),
                    v_edge_vec=torch.tensor(normal_tensor(cfg, 6, (E, 3), dtype=dtype)[perm], **dev).contiguous(),
                    v_phi=torch.tensor(normal_tensor(cfg, 7, (E, K), dtype=dtype)[perm], **dev).contiguous(),
                    v_A=torch.tensor(normal_tensor(cfg, 9, (K, info["n_weights"]), dtype=dtype), **dev))
        if args.radial:   # the radial values' direction follows from the position directions
            del dirs["v_phi"]
        gg = dict(gg_x=torch.empty_like(x), gg_pos=torch.empty_like(pos), gg_edge_vec=torch.empty((E, 3), **dev),
                  gg_phi=torch.empty_like(phi), gg_A=torch.empty_like(A), gg_grad_out=torch.empty_like(out))

    phi_in = None if args.radial else phi
    # Forward + backward: the forward keeps its state for the backward (fully connected: the
    # receiver state S; channelwise: the per-edge coefficient rows of the conventional forward).
    keep_state = "bwd" in passes and not args.recompute_state and (
        "fwds" in passes if spec["mode"] == "uvw" else "fwd" in passes)
    if keep_state:
        try:
            cg.state_size(plan, graph)
        except cg.CgtpError as err:   # rows longer than N_w (high l): the backward recomputes them
            if err.status != 2:
                raise
            keep_state = False
    state = conv.state_buffer() if keep_state else None

    def step():
        for ps in passes:
            if ps in ("fwd", "fwds"):
                sched = cg.CONVENTIONAL if ps == "fwd" else cg.STREAMED
                if keep_state and sched == (cg.STREAMED if spec["mode"] == "uvw" else cg.CONVENTIONAL):
                    cg.conv_forward_keep_state(plan, graph, x, pos, shift, phi_in, A, out, state, ws[ps])
                else:
                    cg.conv_forward(plan, graph, sched, x, pos, shift, phi_in, A, out, ws[ps])
            elif ps == "bwd" and keep_state:
                cg.conv_backward_with_state(plan, graph, x, pos, shift, phi_in, A, gout, state, grad_x=grads["x"],
                                            grad_pos=grads["pos"], grad_edge_vec=grads["edge_vec"],
                                            grad_phi=grads["phi"], grad_A=grads["A"], workspace=ws[ps])
            elif ps == "bwd":
                cg.conv_backward(plan, graph, x, pos, shift, phi_in, A, gout, grad_x=grads["x"], grad_pos=grads["pos"],
                                 grad_edge_vec=grads["edge_vec"], grad_phi=grads["phi"], grad_A=grads["A"],
                                 workspace=ws[ps])
            else:
                cg.conv_double_backward(plan, graph, x, pos, shift, phi_in, A, gout, **dirs, **gg, workspace=ws[ps])

    # Pre-roll: untimed steps for at least PREROLL_MS, so that the W warm-up steps and the K timed
    # steps run at ramped clocks.  Then exactly W warm-up and K timed steps, bracketed by
    # synchronisations; HIP events on the launch stream between the timed steps give per-step
    # durations for the median.
    torch.cuda.synchronize()
    t_pre, n_pre = time.perf_counter(), 0
    while (time.perf_counter() - t_pre) * 1e3 < PREROLL_MS or n_pre < 3:
        step()
        n_pre += 1
        if n_pre % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    preroll_ms = (time.perf_counter() - t_pre) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for k in range(args.steps):
        step()
        ev[k + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = E * args.steps / elapsed
    step_ms = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps))
    median_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])

    # Median protocol of the Sobek page (section 5.1): >= 50 ms of warm-up (the pre-roll and the
    # W steps above), then per-step event samples totalling >= 250 ms (at least 10), median.
    samples = list(step_ms)
    while sum(samples) < PROTOCOL_MIN_MS or len(samples) < PROTOCOL_MIN_SAMPLES:
        batch = [torch.cuda.Event(enable_timing=True) for _ in range(9)]
        batch[0].record()
        for k in range(8):
            step()
            batch[k + 1].record()
        torch.cuda.synchronize()
        samples += [batch[k].elapsed_time(batch[k + 1]) for k in range(8)]
    samples.sort()
    proto_median = samples[len(samples) // 2]
    protocol = {"warmup_ms": round(preroll_ms + args.warmup * ms_per_step, 1), "samples": len(samples),
                "sample_ms_total": round(sum(samples), 1), "median_ms_per_step": round(proto_median, 4),
                "edges_per_s_median": round(E / (proto_median * 1e-3), 1)}

    # Per-kernel durations from HIP events around each launch (a separate region).
    result_kernels, roofline, step_fma = {}, None, 0.0
    if args.profile_steps > 0:
        cg._lib.profile_begin()
        for _ in range(args.profile_steps):
            step()
        torch.cuda.synchronize()
        prof = cg._lib.profile_end()
        fma = kernel_fma(plan, spec, E, N, passes, keep_state)
        step_fma = sum(fma.values())
        for name, (n, ms) in prof.items():
            us_step = 1e3 * ms / args.profile_steps
            entry = {"launches_per_step": n / args.profile_steps, "us_per_step": round(us_step, 2),
                     "avg_us": round(1e3 * ms / n, 2)}
            if name in fma:
                entry["tflops"] = round(2.0 * fma[name] / (us_step * 1e-6) / 1e12, 3)
            result_kernels[name] = entry
        dominant = max(prof, key=lambda k: prof[k][1])
        d = result_kernels[dominant]
        mfma = dominant.startswith("cgtp_gemm")
        peak = PEAK_MFMA_TFLOPS[dtype] if mfma else PEAK_ALU_PUBLISHED_TFLOPS[dtype]
        achieved = d.get("tflops")
        roofline = {"kernel": dominant, "bound": "mfma" if mfma else "alu", "achieved": achieved,
                    "peak": round(peak, 1), "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4) if achieved else None,
                    "traffic": recorded_traffic(dominant) if cfg == DEFAULT_WORKLOAD else None}
        if not mfma and achieved:
            roofline["peak_unpacked_fma"] = round(PEAK_ALU_UNPACKED_TFLOPS, 1)
            roofline["frac_of_unpacked_fma_peak"] = round(achieved / PEAK_ALU_UNPACKED_TFLOPS, 4)
            if not args.no_peak_probe:
                meas = measured_peaks(torch, cg, dtype)
                roofline["measured_peak"] = meas
                roofline["frac_of_measured_fma_peak"] = round(achieved / meas["fma_tflops"], 4)

    desc = {2: "1,024-atom perturbed diamond (4x4x8 cells, a=3.57 A, sigma 0.05 A), cutoff 5 A; "
               "128x0e+128x1o+128x2e -> 128x0e+128x1o+128x2e+128x3o, SH lmax 3, channelwise, "
               "8 Bessel radial functions",
            1: "64 uniform atoms, 6 A periodic cube, cutoff 3 A; 8x0e+8x1o -> 8x0e+8x1o+8x2e, SH lmax 2, "
               "channelwise, 8 Bessel radial functions",
            3: "1,024-atom perturbed diamond, cutoff 5 A; 64x0e+64x1o+64x2e -> 64x0e+64x1o+64x2e+64x3o, "
               "SH lmax 3, channelwise, 8 Bessel radial functions",
            4: "16,384 uniform atoms at 0.1 /A^3, cutoff 5 A; 64x0e+64x1o+64x2e -> same, SH lmax 2, fully "
               "connected (uvw), 8 Bessel radial functions",
            5: "4,096 uniform atoms, 60 expected neighbours within 6 A; 32x(0e..6e) -> same, SH lmax 6, "
               "channelwise, 16 Gaussian radial functions"}[cfg]
    label = " + ".join(PASS_NAMES[p] for p in passes)
    result = {
        "metric": "edges/sec for CGTP conv fwd+bwd, MACE-like irreps, fp32" if cfg == DEFAULT_WORKLOAD
        else f"edges/sec for CGTP conv {label}, {dtype}",
        "value": round(value, 1),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "median_ms_per_step": round(median_ms, 4),
        "preroll": {"steps": n_pre, "ms": round(preroll_ms, 1)},
        "protocol": protocol,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64" if dtype == "float64" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{desc}; {label}" + ("; gradients of x, phi, A and positions" if "bwd" in passes
                                                     else ""),
                   "n_nodes": N, "n_edges": E, "passes": list(passes), "radial_in_kernel": bool(args.radial),
                   **({"receiver_state_kept": keep_state} if spec["mode"] == "uvw" else
                      {"edge_rows_kept": keep_state} if "bwd" in passes else {}),
                   "scratch_budget_mib": args.scratch_mib},
        "gflops_algorithmic": round(2.0 * step_fma / (ms_per_step * 1e-3) / 1e9, 1) if step_fma else None,
        "kernels": result_kernels,
        "roofline": roofline,
    }
    if cfg == DEFAULT_WORKLOAD and not args.no_cpu_baseline and not args.radial:
        result["cpu_baseline"], result["parity"] = cpu_baseline(w, plan, perm, x_h, A_h, g_h, out, grads)
    print(json.dumps(result), flush=True)
    return 0


def channelwise_sweep(torch, cg, args) -> int:
    """Channelwise (uvu) sweeps on the 1,024-atom diamond graph, conventional forward + backward
    (fp32, 8 radial functions): `channels` varies the multiplicity C of the l <= 3 profile
    (C x (0e,1o,2e) -> C x (0e,1o,2e,3o), SH l <= 3); `lmax` varies L with 64 channels
    (64 x (0..L) -> 64 x (0..L), SH l <= L, parities (-1)^l)."""
    from workloads import CONFIGS, make_workload, normal_tensor
    from workloads.sweeps import CHANNEL_POINTS, LMAX_POINTS, channelwise_profile
    cfg = 2
    base = CONFIGS[cfg]
    w = make_workload(cfg)
    points = CHANNEL_POINTS if args.sweep == "channels" else LMAX_POINTS
    if args.points:
        points = [int(v) for v in args.points.split(",")]
    steps, warmup = max(1, min(args.steps, 20)), max(1, min(args.warmup, 3))
    K = base["K"]
    graph = cg.Graph(w.n_nodes, w.recv, w.send, w.image)
    perm = graph.perm
    N, E = w.n_nodes, graph.n_edges
    dev = dict(dtype=torch.float32, device="cuda")
    r32 = lambda a: a.astype(np.float32).astype(np.float64)  # noqa: E731
    pos = torch.tensor(r32(w.pos), **dev)
    shift = torch.tensor(r32(w.shift[perm]), **dev).contiguous()
    phi = torch.tensor(r32(w.phi[perm]), **dev).contiguous()
    graph.upload()
    for pt in points:
        irr_in, irr_sh, irr_out = channelwise_profile(args.sweep, pt)
        spec = dict(base, irreps_in=irr_in, irreps_sh=irr_sh, irreps_out=irr_out)
        plan = cg.Plan(irr_in, irr_sh, irr_out, "uvu", "float32", K)
        plan.compile((cg.OP_FORWARD, cg.OP_BACKWARD))
        info = plan.info
        x = torch.tensor(normal_tensor(cfg, 1, (N, info["c_in"]), dtype="float32"), **dev)
        A = torch.tensor(normal_tensor(cfg, 2, (K, info["n_weights"]), std=1.0 / np.sqrt(K), dtype="float32"), **dev)
        gout = torch.tensor(normal_tensor(cfg, 3, (N, info["c_out"]), dtype="float32"), **dev)
        conv = cg.Convolution(plan, graph)
        ws_f, ws_b = conv.workspace(cg.OP_FORWARD), conv.workspace(cg.OP_BACKWARD)
        out = torch.empty((N, info["c_out"]), **dev)
        grads = dict(x=torch.empty_like(x), pos=torch.empty_like(pos), edge_vec=torch.empty((E, 3), **dev),
                     phi=torch.empty_like(phi), A=torch.empty_like(A))

        def step():
            cg.conv_forward(plan, graph, cg.CONVENTIONAL, x, pos, shift, phi, A, out, ws_f)
            cg.conv_backward(plan, graph, x, pos, shift, phi, A, gout, grad_x=grads["x"], grad_pos=grads["pos"],
                             grad_edge_vec=grads["edge_vec"], grad_phi=grads["phi"], grad_A=grads["A"],
                             workspace=ws_b)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        kernels = {}
        if args.profile_steps > 0:
            cg._lib.profile_begin()
            step()
            torch.cuda.synchronize()
            prof = cg._lib.profile_end()
            fma = kernel_fma(plan, spec, E, N, ("fwd", "bwd"))
            for name, (n, ms) in prof.items():
                entry = {"us": round(1e3 * ms, 2)}
                if name in fma and ms > 0:
                    entry["tflops"] = round(2.0 * fma[name] / (ms * 1e-3) / 1e12, 3)
                    entry["frac"] = round(entry["tflops"] / PEAK_ALU_UNPACKED_TFLOPS, 4)
                kernels[name] = entry
        line = {"sweep": args.sweep, "point": pt, "irreps_in": irr_in, "irreps_out": irr_out,
                "n_paths": info["n_paths"], "n_weights": info["n_weights"], "n_nodes": N, "n_edges": E,
                "ms_fwd_bwd": round(1e3 * dt, 3), "edges_per_s_fwd_bwd": round(E / dt, 1), "steps": steps,
                "kernels": kernels}
        print(json.dumps(line), flush=True)
        del plan, conv, ws_f, ws_b, out, grads, x, A, gout
    return 0


def skew_sweep(torch, cg, args) -> int:
    """Skewed in-degrees (LunaTP section 4.2, "task ordering"): the l <= 3, 128-channel channelwise
    profile (K = 16) on 4,096-node graphs whose receivers draw their expected degree from
    32 exp(sigma z); conventional forward + backward per point, once with the nodes in index order
    and once heaviest first (cgtp_graph_set_order), 1 GiB scratch budget (one receiver chunk)."""
    from workloads import sweeps
    s = sweeps.SKEW_PROFILE
    points = sweeps.SKEW_POINTS if not args.points else [int(v) for v in args.points.split(",")]
    steps, warmup = max(1, min(args.steps, 20)), max(1, min(args.warmup, 5))
    plan = cg.Plan(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"], s["dtype"], s["K"])
    plan.set_scratch_budget(1 << 30)
    plan.compile((cg.OP_FORWARD, cg.OP_BACKWARD))
    info = plan.info
    dev = dict(dtype=torch.float32, device="cuda")
    for pt in points:
        g = sweeps.skew_graph(pt)
        deg = np.bincount(g.recv, minlength=g.n_nodes)
        line = {"sweep": "skew", "point": pt, "sigma": pt / 10.0, "n_nodes": g.n_nodes, "n_edges": g.n_edges,
                "mean_degree": round(float(deg.mean()), 2), "max_degree": int(deg.max()),
                "irreps_in": s["irreps_in"], "steps": steps}
        for order, name in ((0, "index"), (1, "degree")):
            graph = cg.Graph(g.n_nodes, g.recv, g.send, g.image)
            graph.set_order(order)
            perm = graph.perm
            x = torch.tensor(sweeps.normal(1, (g.n_nodes, info["c_in"])), **dev)
            A = torch.tensor(sweeps.normal(2, (s["K"], info["n_weights"]), std=1.0 / np.sqrt(s["K"])), **dev)
            gout = torch.tensor(sweeps.normal(3, (g.n_nodes, info["c_out"])), **dev)
            pos = torch.tensor(g.pos.astype(np.float32), **dev)
            shift = torch.tensor(g.shift[perm].astype(np.float32), **dev).contiguous()
            phi = torch.tensor(g.phi[perm].astype(np.float32), **dev).contiguous()
            graph.upload()
            conv = cg.Convolution(plan, graph)
            ws_f, ws_b = conv.workspace(cg.OP_FORWARD), conv.workspace(cg.OP_BACKWARD)
            out = torch.empty((g.n_nodes, info["c_out"]), **dev)
            grads = dict(x=torch.empty_like(x), pos=torch.empty_like(pos),
                         edge_vec=torch.empty((g.n_edges, 3), **dev), phi=torch.empty_like(phi), A=torch.empty_like(A))

            def step():
                cg.conv_forward(plan, graph, cg.CONVENTIONAL, x, pos, shift, phi, A, out, ws_f)
                cg.conv_backward(plan, graph, x, pos, shift, phi, A, gout, grad_x=grads["x"], grad_pos=grads["pos"],
                                 grad_edge_vec=grads["edge_vec"], grad_phi=grads["phi"], grad_A=grads["A"],
                                 workspace=ws_b)

            for _ in range(warmup):
                step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / steps
            kernels = {}
            if args.profile_steps > 0:
                cg._lib.profile_begin()
                step()
                torch.cuda.synchronize()
                kernels = {k: round(1e3 * ms, 1) for k, (n, ms) in cg._lib.profile_end().items()}
            line[name] = {"ms_fwd_bwd": round(1e3 * dt, 3), "edges_per_s_fwd_bwd": round(g.n_edges / dt, 1),
                          "kernel_us": kernels}
            del graph, conv, ws_f, ws_b, out, grads, x, A, gout, pos, shift, phi
        line["speedup_degree_order"] = round(line["index"]["ms_fwd_bwd"] / line["degree"]["ms_fwd_bwd"], 3)
        print(json.dumps(line), flush=True)
    return 0


def sweep(torch, cg, args) -> int:
    """Scaling axis `args.sweep` of the fully connected profiles: streamed forward and backward
    (gradients of x, phi, A and positions) per point, timed separately with the library's default
    scratch budget."""
    from workloads import sweeps
    if args.sweep in ("channels", "lmax"):
        return channelwise_sweep(torch, cg, args)
    if args.sweep == "skew":
        return skew_sweep(torch, cg, args)

    points = sweeps.DEGREES if args.sweep == "degree" else sweeps.COPIES
    if args.points:
        points = [int(v) for v in args.points.split(",")]
    profiles = [args.profile] if args.profile else sorted(sweeps.PROFILES)
    steps, warmup = max(1, min(args.steps, 5)), max(1, min(args.warmup, 2))
    for L in profiles:
        s = sweeps.PROFILES[L]
        plan = cg.Plan(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"], s["dtype"], s["K"])
        if args.scratch_mib > 0:
            plan.set_scratch_budget(args.scratch_mib << 20)
        plan.compile((cg.OP_FORWARD, cg.OP_BACKWARD))
        info = plan.info
        for pt in points:
            g = sweeps.sweep_graph(args.sweep, pt)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            base = torch.cuda.memory_allocated()
            graph = cg.Graph(g.n_nodes, g.recv, g.send, g.image)
            perm = graph.perm
            N, E = g.n_nodes, graph.n_edges
            dev = dict(dtype=torch.float32, device="cuda")
            x = torch.tensor(sweeps.normal(1, (N, info["c_in"])), **dev)
            A = torch.tensor(sweeps.normal(2, (s["K"], info["n_weights"]), std=1.0 / np.sqrt(s["K"])), **dev)
            gout = torch.tensor(sweeps.normal(3, (N, info["c_out"])), **dev)
            r32 = lambda a: a.astype(np.float32)  # noqa: E731
            pos = torch.tensor(r32(g.pos), **dev)
            shift = torch.tensor(r32(g.shift[perm]), **dev).contiguous()
            phi = torch.tensor(r32(g.phi[perm]), **dev).contiguous()
            graph.upload()
            conv = cg.Convolution(plan, graph)
            ws_f, ws_b = conv.workspace(cg.OP_FORWARD), conv.workspace(cg.OP_BACKWARD)
            out = torch.empty((N, info["c_out"]), **dev)
            grads = dict(x=torch.empty_like(x), pos=torch.empty_like(pos), edge_vec=torch.empty((E, 3), **dev),
                         phi=torch.empty_like(phi), A=torch.empty_like(A))

            def fwd():
                cg.conv_forward(plan, graph, cg.STREAMED, x, pos, shift, phi, A, out, ws_f)

            def bwd():
                cg.conv_backward(plan, graph, x, pos, shift, phi, A, gout, grad_x=grads["x"], grad_pos=grads["pos"],
                                 grad_edge_vec=grads["edge_vec"], grad_phi=grads["phi"], grad_A=grads["A"],
                                 workspace=ws_b)

            times = {}
            for name, fn in (("fwd", fwd), ("bwd", bwd)):
                for _ in range(warmup):
                    fn()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(steps):
                    fn()
                torch.cuda.synchronize()
                times[name] = (time.perf_counter() - t0) / steps
            kernels = {}
            if args.profile_steps > 0:
                cg._lib.profile_begin()
                fwd()
                bwd()
                torch.cuda.synchronize()
                kernels = {k: round(1e3 * ms, 1) for k, (n, ms) in cg._lib.profile_end().items()}
            line = {"sweep": args.sweep, "point": pt, "profile": f"L{L} " + s["irreps_in"], "n_weights": info["n_weights"],
                    "n_nodes": N, "n_edges": E, "mean_degree": round(E / N, 2), "cutoff_A": round(g.rc, 3),
                    "fwd_ms": round(1e3 * times["fwd"], 3), "bwd_ms": round(1e3 * times["bwd"], 3),
                    "edges_per_s_fwd_bwd": round(E / (times["fwd"] + times["bwd"]), 1),
                    "workspace_fwd_bytes": int(ws_f.numel()), "workspace_bwd_bytes": int(ws_b.numel()),
                    "materialized_W_fp32_bytes": 4 * E * info["n_weights"],
                    "peak_alloc_bytes": int(torch.cuda.max_memory_allocated() - base),
                    "scratch_budget_mib": args.scratch_mib or 256, "steps": steps, "kernel_us": kernels}
            print(json.dumps(line), flush=True)
            del graph, conv, ws_f, ws_b, out, grads, x, A, gout, pos, shift, phi
    return 0


COPY_BYTES = 256 << 20


def triple_bench(torch, cg, args, cfg, spec, w, plan, graph):
    """Third-order derivative (cgtp_conv_triple_backward) on a standard workload: one JSON line with
    the time per call (HIP events around each call, median) and edges/s, and per-kernel times."""
    from workloads import normal_tensor
    dtype = spec["dtype"]
    tdt = torch.float64 if dtype == "float64" else torch.float32
    dev = dict(dtype=tdt, device="cuda")
    info = plan.info
    N, E, K = w.n_nodes, graph.n_edges, spec["K"]
    perm = graph.perm
    rnd = (lambda a: a.astype(np.float32).astype(np.float64)) if dtype == "float32" else (lambda a: a)
    # The edge operand: any E x sh_dim values drive the same kernels; seeded N(0, 1) draws stand in
    # for the harmonics (the bench does not evaluate the method's arithmetic on the host).
    shapes = dict(x=(N, info["c_in"]), Y=(E, info["sh_dim"]), phi=(E, K), A=(K, info["n_weights"]),
                  grad_out=(N, info["c_out"]))
    h = dict(x=normal_tensor(cfg, 1, shapes["x"], dtype=dtype), Y=normal_tensor(cfg, 30, shapes["Y"], dtype=dtype),
             phi=rnd(w.phi[perm]), A=normal_tensor(cfg, 2, shapes["A"], std=1.0 / np.sqrt(K), dtype=dtype),
             grad_out=normal_tensor(cfg, 3, shapes["grad_out"], dtype=dtype))
    for s_, name in enumerate(("v_x", "v_Y", "v_phi", "v_A", "q_x", "q_Y", "q_phi", "q_A", "q_grad_out")):
        h[name] = normal_tensor(cfg, 20 + s_, shapes[name[2:]], dtype=dtype)
    t = {k: torch.tensor(np.ascontiguousarray(v), **dev) for k, v in h.items()}
    plan.compile((cg.OP_TRIPLE_BACKWARD,))
    graph.upload()
    conv = cg.Convolution(plan, graph)
    ws = conv.workspace(cg.OP_TRIPLE_BACKWARD)
    outs = {k: torch.empty_like(t[k.replace("v_", "")]) for k in cg._lib.TRIPLE_OUTPUTS}

    def call():
        cg._lib.conv_triple_backward(plan, graph, t, outs, ws)

    for _ in range(max(3, args.warmup)):
        call()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for k in range(args.steps):
        call()
        evs[k + 1].record()
    torch.cuda.synchronize()
    ms = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps))
    med = ms[len(ms) // 2]
    kernels = {}
    cg._lib.profile_begin()
    call()
    torch.cuda.synchronize()
    for name, (n, tot) in cg._lib.profile_end().items():
        kernels[name] = {"launches": n, "us": round(1e3 * tot, 1)}
    line = {"pass": "triple backward", "workload": cfg, "n_nodes": N, "n_edges": E, "dtype": dtype,
            "irreps_in": spec["irreps_in"], "steps": args.steps, "median_ms": round(med, 3),
            "edges_per_s": round(E / (med * 1e-3), 1), "workspace_bytes": int(ws.numel()), "kernel_us": kernels}
    print(json.dumps(line), flush=True)
    return 0


def measured_peaks(torch, cg, dtype):
    """Achievable ceilings on this device from the library's probe kernels: the FMA rate of the
    kernels' precision (no packed fp32) and the copy bandwidth over 2 x 512 MiB (read + write)."""
    lib = cg._lib
    small = torch.zeros(8, dtype=torch.float64, device="cuda")
    kind = lib.PEAK_FMA_F64 if dtype == "float64" else lib.PEAK_FMA_F32
    fma_best, fma_med = lib.measure_peak(kind, small, reps=5)
    src = torch.ones(512 << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    bw_best, bw_med = lib.measure_peak(lib.PEAK_COPY, dst, src, reps=5)
    del src, dst
    return {"fma_tflops": round(fma_best, 2), "fma_tflops_median": round(fma_med, 2),
            "copy_gbs": round(bw_best, 1), "copy_gbs_median": round(bw_med, 1),
            "copy_frac_of_8tbs": round(bw_best / PEAK_HBM_GBS, 4)}


def copy_probe(torch) -> int:
    """Five copies of a 256 MiB buffer: each reads and writes COPY_BYTES of HBM.  The FETCH_SIZE and
    WRITE_SIZE counters of these dispatches, divided by COPY_BYTES, give the factors that turn the
    counters of the convolution kernels into bytes."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_BYTES, "launches": 5}), flush=True)
    return 0


def cpu_baseline(w, plan, perm, x_h, A_h, g_h, out, grads):
    """Oracle forward + backward on a contiguous receiver slice, timed on the host cores.

    The same run compares the slice's GPU results with the oracle (forward rows of the slice's
    receivers; per-edge phi and edge-vector gradients of its edges).
    """
    import torch

    from oracle import conv as oconv
    from oracle import csr as ocsr
    from oracle.irreps import make_problem

    spec = w.spec
    problem = make_problem(spec["irreps_in"], spec["irreps_sh"], spec["irreps_out"], spec["mode"])
    operm, row_ptr, _ = ocsr.receiver_csr(w.n_nodes, w.recv, w.send, w.image)
    n_slice = w.n_nodes // 4
    e_hi = int(row_ptr[n_slice])
    sel = operm[:e_hi]
    recv, send = w.recv[sel], w.send[sel]
    r32 = lambda a: a.astype(np.float32).astype(np.float64)  # noqa: E731
    pos = r32(w.pos)
    shift = r32(w.shift[sel])
    phi = r32(w.phi[sel])
    t0 = time.perf_counter()
    ev = oconv.edge_vectors(pos, shift, recv, send)
    m = oconv.forward_conventional(problem, x_h, ev, recv, send, phi, A_h)
    b = oconv.backward(problem, x_h, ev, recv, send, phi, A_h, g_h, n_nodes=w.n_nodes)
    dt = time.perf_counter() - t0
    times = [dt]
    for _ in range(2):      # median of three runs
        t1 = time.perf_counter()
        ev = oconv.edge_vectors(pos, shift, recv, send)
        oconv.forward_conventional(problem, x_h, ev, recv, send, phi, A_h)
        oconv.backward(problem, x_h, ev, recv, send, phi, A_h, g_h, n_nodes=w.n_nodes)
        times.append(time.perf_counter() - t1)
    times.sort()
    dt_med = times[1]
    rel = lambda a, r: float(np.abs(a - r).max() / np.abs(r).max())  # noqa: E731
    # x-bar and pos-bar of 8 seeded nodes: the oracle backward over every edge that touches them
    # (their in- and out-edges), outside the timed baseline.
    inside = np.unique(np.random.default_rng(2).choice(w.n_nodes, 8, replace=False))
    touch = np.nonzero(np.isin(w.recv[operm], inside) | np.isin(w.send[operm], inside))[0]
    te = operm[touch]
    bn = oconv.backward(problem, x_h, oconv.edge_vectors(pos, r32(w.shift[te]), w.recv[te], w.send[te]),
                        w.recv[te], w.send[te], r32(w.phi[te]), A_h, g_h, n_nodes=w.n_nodes)
    parity = {
        "forward_rows": rel(out.cpu().numpy()[:n_slice], m.numpy()[:n_slice]),
        "grad_phi_edges": rel(grads["phi"].cpu().numpy()[:e_hi], b["phi"].numpy()),
        "grad_edge_vec_edges": rel(grads["edge_vec"].cpu().numpy()[:e_hi], b["edge_vec"].numpy()),
        "grad_x_nodes": rel(grads["x"].cpu().numpy()[inside], bn["x"].numpy()[inside]),
        "grad_pos_nodes": rel(grads["pos"].cpu().numpy()[inside], bn["pos"].numpy()[inside]),
        "nodes_checked": [int(v) for v in inside],
        "tolerance": 1e-5,
    }
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    baseline = {"value": round(e_hi / dt_med, 1), "unit": "edges/s", "cores": torch.get_num_threads(),
                "kind": "oracle",
                "sample": f"receivers 0..{n_slice - 1} of the workload with their {e_hi} incoming edges, "
                          f"float64 forward + backward, median of 3 runs ({', '.join(f'{t:.1f}' for t in times)} s)",
                "host_cpus": os.cpu_count(), "cpu_model": cpu_model,
                "threads_env": {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "MKL_NUM_THREADS")}}
    assert np.array_equal(perm[:e_hi], sel), "library and oracle CSR orders differ"
    return baseline, parity


if __name__ == "__main__":
    sys.exit(main())
