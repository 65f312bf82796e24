"""Channelwise convolution with blocks of different multiplicities (needs an MI355X).

The input irreps are LunaTP's C3 profile (Table 1: 128x0e+64x1o+32x2e+32x3o with SH up to l = 3),
outputs the same blocks.  Channelwise paths join blocks of equal multiplicity, so the blocks need
2, 1, 1 and 1 channel blocks of 64 lanes (the 32-channel blocks fill half a wave): workgroups
that run every channel block of a feature block carry idle waves for the smaller blocks.  Also a
second profile with a 160-channel block (a ragged third channel block) next to 64-channel ones.
"""

from __future__ import annotations

import pytest

from oracle import conv
from tests.oracle_helpers import effective_edge_direction, make_case, make_directions

pytestmark = pytest.mark.gpu

C3 = dict(irreps_in="128x0e+64x1o+32x2e+32x3o", irreps_sh="1x0e+1x1o+1x2e+1x3o",
          irreps_out="128x0e+64x1o+32x2e+32x3o")
WIDE = dict(irreps_in="160x0e+64x1o+64x2e", irreps_sh="1x0e+1x1o+1x2e",
            irreps_out="160x0e+64x1o+64x2e+160x2e")
KEYS = ("x", "pos", "edge_vec", "phi", "A")


def _gpu(case):
    from tests.gpu_helpers import GpuCase
    return GpuCase(case)


def _cmp(got, ref, dtype, keys, label):
    from tests.gpu_helpers import TOL, rel_err
    for k in keys:
        err = rel_err(got[k].cpu().numpy()[:len(ref[k])], ref[k].numpy())
        print(f"{label} {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL[dtype], (k, err)


@pytest.mark.parametrize("profile", ["C3", "WIDE"])
@pytest.mark.parametrize("dtype", ["float32", "float64"])
def test_hetero_forward_backward(profile, dtype):
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(1, irreps_override=C3 if profile == "C3" else WIDE, dtype=dtype)
    g = _gpu(case)
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    for sched, name in ((_lib.CONVENTIONAL, "conventional"), (_lib.STREAMED, "streamed")):
        err = rel_err(g.forward(sched).cpu().numpy(), ref)
        print(f"{profile} {dtype} forward {name}: rel err {err:.3e}", flush=True)
        assert err <= TOL[dtype], name
    b = conv.backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A, case.grad_out)
    _cmp(g.backward(), b, dtype, KEYS, f"{profile} {dtype} grad")


@pytest.mark.parametrize("profile", ["C1", "C5", "C7", "C9"])
def test_lunatp_profiles_forward_backward(profile):
    """LunaTP's mixed-multiplicity cases (Appendix A.1): C5 (l <= 4, a 320-channel scalar block:
    five channel blocks, the last ragged), C7 (l <= 5), C9 (l <= 6, 32-channel blocks on half
    waves) and C1 (edge block 1 labelled 1e, so all paths are even), fp32 on the 64-atom graph:
    both forward schedules and every gradient against the oracle."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    from workloads.sweeps import lunatp_profile
    case = make_case(1, irreps_override=lunatp_profile(profile), dtype="float32")
    g = _gpu(case)
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    for sched, name in ((_lib.CONVENTIONAL, "conventional"), (_lib.STREAMED, "streamed")):
        err = rel_err(g.forward(sched).cpu().numpy(), ref)
        print(f"{profile} forward {name}: rel err {err:.3e} ({len(case.problem.paths)} paths)", flush=True)
        assert err <= TOL["float32"], name
    b = conv.backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A, case.grad_out)
    _cmp(g.backward(), b, "float32", KEYS, f"{profile} grad")


@pytest.mark.parametrize("dtype", ["float32", "float64"])
def test_hetero_double_backward(dtype):
    case = make_case(1, irreps_override=C3, dtype=dtype)
    dirs = make_directions(case)
    v_e = effective_edge_direction(case, dirs.get("v_edge_vec"), dirs.get("v_pos"))
    ref = conv.double_backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A,
                               case.grad_out, v_x=dirs.get("v_x"), v_e=v_e, v_phi=dirs.get("v_phi"),
                               v_A=dirs.get("v_A"))
    _cmp(_gpu(case).double_backward(dirs), ref, dtype, KEYS + ("grad_out",), f"C3 {dtype} gg")


@pytest.mark.parametrize("dtype", ["float32", "float64"])
def test_layout_convert_matches_block_transpose(dtype):
    """ir_mul <-> mul_ir per block (a permutation: bit-exact), both sides, round trip."""
    import numpy as np
    import torch
    from clebsch_gordan_tensor_receiver_amd import _lib
    spec = C3
    plan = _lib.Plan(spec["irreps_in"], spec["irreps_sh"], spec["irreps_out"], "uvu", dtype, 8)
    for side, irreps in ((0, spec["irreps_in"]), (1, spec["irreps_out"])):
        blocks = [(int(t.split("x")[0]), int(t.split("x")[1][:-1])) for t in irreps.split("+")]
        width = sum(m * (2 * l + 1) for m, l in blocks)
        n = 37
        h = np.random.default_rng(side).normal(size=(n, width))
        want = np.empty_like(h)   # mul_ir of h read as ir_mul
        off = 0
        for m, l in blocks:
            d = 2 * l + 1
            want[:, off:off + m * d] = h[:, off:off + m * d].reshape(n, d, m).transpose(0, 2, 1).reshape(n, m * d)
            off += m * d
        dt = torch.float64 if dtype == "float64" else torch.float32
        src = torch.tensor(h, dtype=dt, device="cuda")
        mid = torch.empty_like(src)
        back = torch.empty_like(src)
        _lib.layout_convert(plan, side, 1, src, mid)
        _lib.layout_convert(plan, side, 0, mid, back)
        torch.cuda.synchronize()
        assert np.array_equal(mid.cpu().numpy(), want.astype(src.cpu().numpy().dtype))
        assert np.array_equal(back.cpu().numpy(), src.cpu().numpy())


@pytest.mark.parametrize("profile", ["C1", "C5", "C7", "C9"])
def test_lunatp_profiles_double_backward(profile):
    """Double backward on LunaTP's mixed-multiplicity cases (Appendix A.1; the page quotes its
    largest double-backward gain on C9), fp32 on the 64-atom graph: every output against the
    oracle."""
    from tests.test_gpu_double_backward import _compare as dcompare, _oracle as doracle
    from workloads.sweeps import lunatp_profile
    case = make_case(1, irreps_override=lunatp_profile(profile), dtype="float32")
    dirs = make_directions(case)
    dcompare(_gpu(case).double_backward(dirs), doracle(case, dirs), "float32", label=f"{profile}")


@pytest.mark.parametrize("profile", ["C1", "C5", "C7", "C9"])
def test_lunatp_profiles_triple_backward(profile):
    """Third-order derivative (LunaTP Appendix F, Algorithm 4) on the mixed-multiplicity cases,
    fp32 on the 64-atom graph: every output against the oracle."""
    from tests.test_gpu_triple_backward import _compare as tcompare, _gpu_run, _inputs, _oracle as toracle
    from workloads.sweeps import lunatp_profile
    case = make_case(1, irreps_override=lunatp_profile(profile), dtype="float32")
    h = _inputs(case)
    _, got = _gpu_run(case, h)
    tcompare(got, toracle(case, h), "float32", f"{profile} triple")
