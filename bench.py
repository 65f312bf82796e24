"""Throughput of the Clebsch-Gordan tensor-product convolution on one MI355X.

One step = forward + backward (gradients of x, phi, A and the positions) of the channelwise
convolution on the 1,024-atom perturbed-diamond graph (cutoff 5 A, ~91k directed edges),
128x0e+128x1o+128x2e -> 128x(0e,1o,2e,3o), SH lmax 3, 8 radial functions, float32, inputs
resident in device memory.  Prints one JSON line:

  metric / value / unit      edges per second of forward + backward (whole job, one GPU)
  roofline                   the dominant kernel against the fp32 vector-ALU peak, from HIP
                             events recorded around every launch inside this process
  cpu_baseline               the float64 CPU oracle on a bounded receiver slice of the same
                             workload, timed on this host (a reported baseline, not a target)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CONFIG = 2
# Non-packed FP32 vector FMA peak: 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz.  The build
# keeps packed FP32 off, so this (not the 157.3 TFLOP/s packed figure) bounds the VALU kernels.
PEAK_FP32_ALU_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
PEAK_FP64_ALU_TFLOPS = 78.6


def algorithmic_fma(plan, n_edges: int, n_nodes: int):
    """FMA per launch of each kernel (one launch covers every edge), from the plan's path table.

    Per path pi with C channels, K radial functions, gnz (m1, m3) pairs, p12 (m1, m2) pairs,
    nnz CG terms and component counts d1, d2, d3:
      forward     C (K + gnz + min(d1, d3)) per edge (w = phi A, T = G x, w applied on the smaller side)
      source bwd  the same per edge (x-bar = w G^T mbar)
      receiver bwd the cheaper of two exact forms: with T = G x, C (2 gnz + 3K + d3) per edge plus
                  2 nnz per edge for Y-bar; or folded through R = sum c mbar (formed once per receiver,
                  C nnz), C (p12 + 2 d2 + 3K) per edge (Q = x R, h = Y.Q, Y-bar += w Q, and the three K
                  contractions w, phi-bar, A-bar)
      prep        nnz per edge (G = sum c Y)
    """
    K = plan.info["num_radial"]
    E, N = n_edges, n_nodes
    deg = E / max(N, 1)
    fwd = recv = prep = 0.0
    for k in range(plan.info["n_paths"]):
        d = plan.path(k)
        idx, _ = plan.cg_table(k)
        gnz = len({(int(a), int(c)) for a, _, c in idx})
        p12 = len({(int(a), int(b)) for a, b, _ in idx})
        nnz = len(idx)
        d1, d2, d3 = 2 * d["l1"] + 1, 2 * d["l2"] + 1, 2 * d["l3"] + 1
        C = d["n_weights"]  # channelwise: one weight per channel
        fwd += C * (K + gnz + min(d1, d3))
        plain = C * (2 * gnz + 3 * K + d3) + 2 * nnz
        fold = C * (p12 + 2 * d2 + 3 * K) + C * nnz / deg
        recv += min(plain, fold)
        prep += nnz
    return {"cgtp_fwd": fwd * E, "cgtp_prep": prep * E, "cgtp_bwd_recv": recv * E, "cgtp_bwd_src": fwd * E}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--profile-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of known size (calibrates the HBM byte counters)")
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
    spec = CONFIGS[CONFIG]
    w = make_workload(CONFIG)
    plan = cg.Plan(spec["irreps_in"], spec["irreps_sh"], spec["irreps_out"], spec["mode"], spec["dtype"], spec["K"])
    graph = cg.Graph(w.n_nodes, w.recv, w.send, w.image)
    perm = graph.perm
    info = plan.info
    K = spec["K"]
    dev = dict(dtype=torch.float32, device="cuda")
    x_h = normal_tensor(CONFIG, 1, (w.n_nodes, info["c_in"]), dtype="float32")
    A_h = normal_tensor(CONFIG, 2, (K, info["n_weights"]), std=1.0 / np.sqrt(K), dtype="float32")
    g_h = normal_tensor(CONFIG, 3, (w.n_nodes, info["c_out"]), dtype="float32")
    x = torch.tensor(x_h, **dev)
    A = torch.tensor(A_h, **dev)
    gout = torch.tensor(g_h, **dev)
    pos = torch.tensor(w.pos.astype(np.float32), **dev)
    shift = torch.tensor(w.shift[perm].astype(np.float32), **dev).contiguous()
    phi = torch.tensor(w.phi[perm].astype(np.float32), **dev).contiguous()
    conv = cg.Convolution(plan, graph)
    plan.compile((cg.OP_FORWARD, cg.OP_BACKWARD))
    graph.upload()
    E = graph.n_edges

    out = torch.empty((w.n_nodes, info["c_out"]), **dev)
    grads = dict(x=torch.empty_like(x), pos=torch.empty_like(pos), edge_vec=torch.empty((E, 3), **dev),
                 phi=torch.empty_like(phi), A=torch.empty_like(A))
    ws_f = conv.workspace(cg.OP_FORWARD)
    ws_b = conv.workspace(cg.OP_BACKWARD)

    def step():
        cg.conv_forward(plan, graph, cg.CONVENTIONAL, x, pos, shift, phi, A, out, ws_f)
        cg.conv_backward(plan, graph, x, pos, shift, phi, A, gout, grad_x=grads["x"], grad_pos=grads["pos"],
                         grad_edge_vec=grads["edge_vec"], grad_phi=grads["phi"], grad_A=grads["A"],
                         workspace=ws_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = E * args.steps / elapsed

    # Per-kernel durations from HIP events around each launch (separate region).
    cg._lib.profile_begin()
    for _ in range(args.profile_steps):
        step()
    torch.cuda.synchronize()
    prof = cg._lib.profile_end()
    fma = algorithmic_fma(plan, E, w.n_nodes)
    kernels = {}
    for name, (n, ms) in prof.items():
        avg_us = 1e3 * ms / n
        entry = {"launches_per_step": n / args.profile_steps, "avg_us": round(avg_us, 2)}
        if name in fma:
            flop = 2.0 * fma[name]  # one launch covers every edge (single receiver chunk)
            entry["tflops"] = round(flop / (avg_us * 1e-6) / 1e12, 3)
        kernels[name] = entry
    dominant = max(prof, key=lambda k: prof[k][1])
    d_entry = kernels[dominant]
    achieved = d_entry.get("tflops")
    roofline = {"kernel": dominant, "bound": "alu", "achieved": achieved, "peak": round(PEAK_FP32_ALU_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_ALU_TFLOPS, 4) if achieved else None,
                "traffic": None}
    step_flop = 2.0 * (fma["cgtp_fwd"] + 2 * fma["cgtp_prep"] + fma["cgtp_bwd_recv"] + fma["cgtp_bwd_src"])

    result = {
        "metric": "edges/sec for CGTP conv fwd+bwd, MACE-like irreps, fp32",
        "value": round(value, 1),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "1,024-atom perturbed diamond (4x4x8 cells, a=3.57 A, sigma 0.05 A), cutoff 5 A; "
                               "128x0e+128x1o+128x2e -> 128x0e+128x1o+128x2e+128x3o, SH lmax 3, channelwise, "
                               "8 Bessel radial functions; forward + backward (x, phi, A, positions)",
                   "n_nodes": w.n_nodes, "n_edges": E, "schedule": "conventional (per-edge weights in registers)"},
        "gflops_algorithmic": round(step_flop / (ms_per_step * 1e-3) / 1e9, 1),
        "kernels": kernels,
        "roofline": roofline,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(w, plan, perm, x_h, A_h, g_h, out, grads)
    print(json.dumps(result), flush=True)
    return 0


COPY_BYTES = 256 << 20


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
    rel = lambda a, r: float(np.abs(a - r).max() / np.abs(r).max())  # noqa: E731
    parity = {
        "forward_rows": rel(out.cpu().numpy()[:n_slice], m.numpy()[:n_slice]),
        "grad_phi_edges": rel(grads["phi"].cpu().numpy()[:e_hi], b["phi"].numpy()),
        "grad_edge_vec_edges": rel(grads["edge_vec"].cpu().numpy()[:e_hi], b["edge_vec"].numpy()),
        "tolerance": 1e-5,
    }
    baseline = {"value": round(e_hi / dt, 1), "unit": "edges/s", "cores": torch.get_num_threads(), "kind": "oracle",
                "sample": f"receivers 0..{n_slice - 1} of the workload with their {e_hi} incoming edges, "
                          f"float64 forward + backward, {dt:.1f} s", "host_cpus": os.cpu_count()}
    assert np.array_equal(perm[:e_hi], sel), "library and oracle CSR orders differ"
    return baseline, parity


if __name__ == "__main__":
    sys.exit(main())
