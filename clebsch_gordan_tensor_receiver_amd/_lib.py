"""ctypes binding of ``libcgtp.so`` (argument marshalling only).

Every computation runs in the library's HIP kernels; torch tensors are used only to own
device memory and to name the current HIP stream.  If the library is missing or fails to
load, every entry point raises: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcgtp.so")

CHANNELWISE, FULLY_CONNECTED = 0, 1
F32, F64 = 0, 1
STREAMED, CONVENTIONAL = 0, 1
DEGENERATE_EDGE = 4
OP_FORWARD, OP_BACKWARD, OP_DOUBLE_BACKWARD, OP_TRIPLE_BACKWARD = 0, 1, 2, 3

EXPORTED = [
    "cgtp_plan_create", "cgtp_plan_destroy", "cgtp_plan_info", "cgtp_plan_path", "cgtp_plan_cg_table",
    "cgtp_plan_compile", "cgtp_plan_set_scratch_budget", "cgtp_plan_set_radial", "cgtp_graph_build", "cgtp_graph_export",
    "cgtp_graph_dims", "cgtp_graph_upload", "cgtp_graph_destroy", "cgtp_workspace_size",
    "cgtp_conv_forward", "cgtp_conv_backward", "cgtp_conv_double_backward", "cgtp_check_edges", "cgtp_layout_convert", "cgtp_error_string", "cgtp_last_error",
    "cgtp_state_size", "cgtp_conv_forward_keep_state", "cgtp_conv_backward_with_state",
    "cgtp_profile_begin", "cgtp_profile_end", "cgtp_profile_count", "cgtp_profile_get", "cgtp_measure_peak",
    "cgtp_conv_forward_static", "cgtp_graph_set_order", "cgtp_conv_triple_backward",
]


class CgtpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"cgtp status {status}: {message}")
        self.status = status


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "n_paths", "n_weights", "c_in", "c_out", "sh_dim", "lmax_sh", "num_radial", "mode", "dtype",
        "n_in_blocks", "n_out_blocks", "cg_nnz", "g_nnz")]


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run clebsch_gordan_tensor_receiver_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z, V = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    ip = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "cgtp_plan_create": [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p, I, I, I, ctypes.POINTER(P)],
        "cgtp_plan_destroy": [P],
        "cgtp_plan_info": [P, ctypes.POINTER(PlanInfo)],
        "cgtp_plan_path": [P, I, ip],
        "cgtp_plan_cg_table": [P, I, ip, ctypes.POINTER(ctypes.c_double), I, ctypes.POINTER(ctypes.c_int)],
        "cgtp_plan_compile": [P, I],
        "cgtp_plan_set_scratch_budget": [P, Z],
        "cgtp_plan_set_radial": [P, ctypes.c_int, ctypes.c_double],
        "cgtp_graph_build": [I, I, ip, ip, ip, ip, ctypes.POINTER(P)],
        "cgtp_graph_export": [P, ip, ip, ip, ip],
        "cgtp_graph_dims": [P, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)],
        "cgtp_graph_upload": [P],
        "cgtp_graph_set_order": [P, I],
        "cgtp_graph_destroy": [P],
        "cgtp_workspace_size": [P, P, I, ctypes.POINTER(Z)],
        "cgtp_conv_forward": [P, P, I, V, V, V, V, V, V, V, Z, V],
        "cgtp_conv_backward": [P, P, V, V, V, V, V, V, V, V, V, V, V, V, Z, V],
        "cgtp_conv_double_backward": [P, P] + [V] * 18 + [Z, V],
        "cgtp_conv_triple_backward": [P, P] + [V] * 24 + [Z, V],
        "cgtp_state_size": [P, P, ctypes.POINTER(Z)],
        "cgtp_conv_forward_keep_state": [P, P, V, V, V, V, V, V, V, Z, V, Z, V],
        "cgtp_conv_backward_with_state": [P, P, V, V, V, V, V, V, V, Z, V, V, V, V, V, V, Z, V],
        "cgtp_check_edges": [P, P, V, V, V, Z, V, ctypes.POINTER(ctypes.c_int)],
        "cgtp_layout_convert": [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, V, V, V],
        "cgtp_profile_begin": [],
        "cgtp_profile_end": [],
        "cgtp_profile_count": [],
        "cgtp_profile_get": [I, ctypes.c_char_p, I, ctypes.POINTER(ctypes.c_longlong),
                             ctypes.POINTER(ctypes.c_double)],
        "cgtp_measure_peak": [I, V, V, Z, I, V, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)],
        "cgtp_conv_forward_static": [P, P, I, V, V, V, V, V, V, V],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.cgtp_error_string.argtypes = [ctypes.c_int]
    lib.cgtp_error_string.restype = ctypes.c_char_p
    lib.cgtp_last_error.argtypes = []
    lib.cgtp_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != 0:
        lib = load()
        raise CgtpError(status, f"{lib.cgtp_error_string(status).decode()}: {lib.cgtp_last_error().decode()}")


def _i32(a: Optional[np.ndarray]):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _ptr(t) -> Optional[int]:
    """Device address of a torch tensor (None stays NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


class Plan:
    def __init__(self, irreps_in: str, irreps_sh: str, irreps_out: str, mode: str = "uvu",
                 dtype: str = "float32", num_radial: int = 8):
        lib = load()
        h = ctypes.c_void_p()
        m = {"uvu": CHANNELWISE, "uvw": FULLY_CONNECTED}[mode]
        d = {"float32": F32, "float64": F64}[dtype]
        check(lib.cgtp_plan_create(irreps_in.encode(), irreps_sh.encode(), irreps_out.encode(), m, d,
                                   int(num_radial), ctypes.byref(h)))
        self.handle = h
        self.dtype = dtype
        self.mode = mode
        info = PlanInfo()
        check(lib.cgtp_plan_info(h, ctypes.byref(info)))
        self.info = {n: getattr(info, n) for n, _ in PlanInfo._fields_}

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.cgtp_plan_destroy(h)
            self.handle = None

    def path(self, k: int):
        desc = np.zeros(9, dtype=np.int32)
        check(load().cgtp_plan_path(self.handle, k, desc.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return dict(zip(("i_in", "i_sh", "i_out", "l1", "l2", "l3", "weight_offset", "n_weights", "cg_nnz"),
                        desc.tolist()))

    def cg_table(self, k: int):
        lib = load()
        n = ctypes.c_int()
        check(lib.cgtp_plan_cg_table(self.handle, k, None, None, 0, ctypes.byref(n)))
        idx = np.zeros((n.value, 3), dtype=np.int32)
        val = np.zeros(n.value, dtype=np.float64)
        check(lib.cgtp_plan_cg_table(self.handle, k, idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     val.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), n.value, ctypes.byref(n)))
        return idx, val

    def compile(self, ops=(OP_FORWARD,)) -> None:
        mask = 0
        for o in ops:
            mask |= 1 << o
        check(load().cgtp_plan_compile(self.handle, mask))

    def set_scratch_budget(self, nbytes: int) -> None:
        check(load().cgtp_plan_set_scratch_budget(self.handle, int(nbytes)))

    def set_radial(self, kind: int, r_cut: float) -> None:
        """Compute phi from |r| in the kernels (1 Bessel + envelope, 2 Gaussian, 0 none); the
        convolution calls then take phi=None."""
        check(load().cgtp_plan_set_radial(self.handle, int(kind), float(r_cut)))


class Graph:
    def __init__(self, n_nodes: int, recv, send, image=None):
        lib = load()
        recv, rp = _i32(recv)
        send, sp = _i32(send)
        image, ip = _i32(None if image is None else np.asarray(image).reshape(-1))
        self.n_nodes = int(n_nodes)
        self.n_edges = int(len(recv))
        self.perm = np.zeros(self.n_edges, dtype=np.int32)
        h = ctypes.c_void_p()
        check(lib.cgtp_graph_build(self.n_nodes, self.n_edges, rp, sp, ip,
                                   self.perm.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.cgtp_graph_destroy(h)
            self.handle = None

    def export(self):
        n, e = self.n_nodes, self.n_edges
        rp = np.zeros(n + 1, np.int32)
        col = np.zeros(max(e, 1), np.int32)
        sp = np.zeros(n + 1, np.int32)
        se = np.zeros(max(e, 1), np.int32)
        P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))  # noqa: E731
        check(load().cgtp_graph_export(self.handle, P(rp), P(col), P(sp), P(se)))
        return rp, col[:e], sp, se[:e]

    def upload(self) -> None:
        check(load().cgtp_graph_upload(self.handle))

    def set_order(self, mode: int) -> None:
        """Node dispatch order (before upload): 0 index, 1 by degree, 2 automatic (default)."""
        check(load().cgtp_graph_set_order(self.handle, int(mode)))


def profile_begin() -> None:
    check(load().cgtp_profile_begin())


def profile_end():
    """Stop launch timing; returns {kernel name: (launches, total ms)}."""
    lib = load()
    check(lib.cgtp_profile_end())
    out = {}
    for k in range(lib.cgtp_profile_count()):
        buf = ctypes.create_string_buffer(128)
        n = ctypes.c_longlong()
        ms = ctypes.c_double()
        check(lib.cgtp_profile_get(k, buf, 128, ctypes.byref(n), ctypes.byref(ms)))
        out[buf.value.decode()] = (int(n.value), float(ms.value))
    return out


PEAK_FMA_F32, PEAK_FMA_F64, PEAK_COPY = 0, 1, 2


def measure_peak(kind: int, dst, src=None, reps: int = 5, stream=None):
    """Measured device ceiling (cgtp_measure_peak): (best, median) in TFLOP/s (kinds 0, 1) or GB/s
    (kind 2, a copy of src into dst, both device tensors of the same byte size)."""
    best, med = ctypes.c_double(), ctypes.c_double()
    nbytes = dst.numel() * dst.element_size()
    check(load().cgtp_measure_peak(int(kind), _ptr(dst), _ptr(src), nbytes if kind == PEAK_COPY else 0, int(reps),
                                   _stream(stream), ctypes.byref(best), ctypes.byref(med)))
    return float(best.value), float(med.value)


def workspace_size(plan: Plan, graph: Graph, op: int) -> int:
    n = ctypes.c_size_t()
    check(load().cgtp_workspace_size(plan.handle, graph.handle, op, ctypes.byref(n)))
    return int(n.value)


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def conv_forward(plan: Plan, graph: Graph, schedule: int, x, pos, shift, phi, A, out, workspace, stream=None):
    check(load().cgtp_conv_forward(plan.handle, graph.handle, schedule, _ptr(x), _ptr(pos), _ptr(shift), _ptr(phi),
                                   _ptr(A), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


def conv_forward_static(plan: Plan, graph: Graph, schedule: int, x, pos, shift, phi, A, out, stream=None):
    """cgtp_conv_forward_static: the forward with the library's static device scratch (no workspace)."""
    check(load().cgtp_conv_forward_static(plan.handle, graph.handle, schedule, _ptr(x), _ptr(pos), _ptr(shift),
                                          _ptr(phi), _ptr(A), _ptr(out), _stream(stream)))


def conv_backward(plan: Plan, graph: Graph, x, pos, shift, phi, A, grad_out, grad_x=None, grad_pos=None,
                  grad_edge_vec=None, grad_phi=None, grad_A=None, workspace=None, stream=None):
    check(load().cgtp_conv_backward(plan.handle, graph.handle, _ptr(x), _ptr(pos), _ptr(shift), _ptr(phi), _ptr(A),
                                    _ptr(grad_out), _ptr(grad_x), _ptr(grad_pos), _ptr(grad_edge_vec),
                                    _ptr(grad_phi), _ptr(grad_A), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))


def state_size(plan: Plan, graph: Graph) -> int:
    n = ctypes.c_size_t()
    check(load().cgtp_state_size(plan.handle, graph.handle, ctypes.byref(n)))
    return n.value


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def conv_forward_keep_state(plan: Plan, graph: Graph, x, pos, shift, phi, A, out, state, workspace, stream=None):
    check(load().cgtp_conv_forward_keep_state(plan.handle, graph.handle, _ptr(x), _ptr(pos), _ptr(shift), _ptr(phi),
                                              _ptr(A), _ptr(out), _ptr(state), _nbytes(state), _ptr(workspace),
                                              _nbytes(workspace), _stream(stream)))


def conv_backward_with_state(plan: Plan, graph: Graph, x, pos, shift, phi, A, grad_out, state, grad_x=None,
                             grad_pos=None, grad_edge_vec=None, grad_phi=None, grad_A=None, workspace=None,
                             stream=None):
    check(load().cgtp_conv_backward_with_state(
        plan.handle, graph.handle, _ptr(x), _ptr(pos), _ptr(shift), _ptr(phi), _ptr(A), _ptr(grad_out), _ptr(state),
        _nbytes(state), _ptr(grad_x), _ptr(grad_pos), _ptr(grad_edge_vec), _ptr(grad_phi), _ptr(grad_A),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def conv_double_backward(plan: Plan, graph: Graph, x, pos, shift, phi, A, grad_out, v_x=None, v_pos=None,
                         v_edge_vec=None, v_phi=None, v_A=None, gg_x=None, gg_pos=None, gg_edge_vec=None,
                         gg_phi=None, gg_A=None, gg_grad_out=None, workspace=None, stream=None):
    check(load().cgtp_conv_double_backward(
        plan.handle, graph.handle, _ptr(x), _ptr(pos), _ptr(shift), _ptr(phi), _ptr(A), _ptr(grad_out),
        _ptr(v_x), _ptr(v_pos), _ptr(v_edge_vec), _ptr(v_phi), _ptr(v_A), _ptr(gg_x), _ptr(gg_pos),
        _ptr(gg_edge_vec), _ptr(gg_phi), _ptr(gg_A), _ptr(gg_grad_out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


TRIPLE_INPUTS = ("x", "Y", "phi", "A", "grad_out", "v_x", "v_Y", "v_phi", "v_A", "q_x", "q_Y", "q_phi", "q_A",
                 "q_grad_out")
TRIPLE_OUTPUTS = ("x", "Y", "phi", "A", "grad_out", "v_x", "v_Y", "v_phi", "v_A")


def conv_triple_backward(plan: Plan, graph: Graph, inputs: dict, outputs: dict, workspace, stream=None):
    """cgtp_conv_triple_backward: `inputs` maps TRIPLE_INPUTS names to device tensors (missing
    directions / cotangents = zero), `outputs` maps TRIPLE_OUTPUTS names to device tensors to fill."""
    args = [_ptr(inputs.get(k)) for k in TRIPLE_INPUTS] + [_ptr(outputs.get(k)) for k in TRIPLE_OUTPUTS]
    check(load().cgtp_conv_triple_backward(plan.handle, graph.handle, *args, _ptr(workspace), _nbytes(workspace),
                                           _stream(stream)))


def layout_convert(plan: Plan, side: int, direction: int, src, dst, stream=None) -> None:
    """Feature layout conversion: side 0 input / 1 output features, direction 0 mul_ir -> ir_mul,
    1 ir_mul -> mul_ir; src and dst are device tensors of shape (N, width)."""
    check(load().cgtp_layout_convert(plan.handle, side, direction, int(src.shape[0]), _ptr(src), _ptr(dst),
                                      _stream(stream)))


def check_edges(plan: Plan, graph: Graph, pos, shift, workspace, stream=None) -> int:
    """Smallest receiver-sorted index of a zero-length edge, or -1 (synchronises the stream)."""
    first = ctypes.c_int(-1)
    st = load().cgtp_check_edges(plan.handle, graph.handle, _ptr(pos), _ptr(shift), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream), ctypes.byref(first))
    if st == DEGENERATE_EDGE:
        return int(first.value)
    check(st)
    return -1


class Convolution:
    """A plan, a graph and a workspace bound together, called with torch device tensors.

    Per-edge inputs (shift, phi) must already be in the graph's receiver-sorted order
    (``graph.perm`` maps sorted positions to the caller's edge indices).
    """

    def __init__(self, plan: Plan, graph: Graph):
        import torch
        self.plan, self.graph = plan, graph
        self.torch_dtype = torch.float64 if plan.dtype == "float64" else torch.float32
        self._ws = {}

    def workspace(self, op: int):
        import torch
        n = workspace_size(self.plan, self.graph, op)
        ws = self._ws.get(op)
        if ws is None or ws.numel() < n:
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
            self._ws[op] = ws
        return ws

    def state_buffer(self):
        """Device buffer for the state kept by forward(..., state=...): the receiver state of a
        fully connected plan, or the per-edge coefficient rows of a channelwise one."""
        import torch
        return torch.empty(state_size(self.plan, self.graph), dtype=torch.uint8, device="cuda")

    def forward(self, x, pos, shift, phi, A, schedule: int = CONVENTIONAL, out=None, state=None):
        """With `state`: also keep the state for backward(); fully connected plans keep it in the
        streamed schedule, channelwise plans in the conventional one (ValueError otherwise)."""
        import torch
        if state is not None:
            keeps = STREAMED if self.plan.info["mode"] == FULLY_CONNECTED else CONVENTIONAL
            if schedule != keeps:
                raise ValueError("this plan keeps its state in the "
                                 + ("streamed" if keeps == STREAMED else "conventional") + " forward only")
        if out is None:
            out = torch.empty((self.graph.n_nodes, self.plan.info["c_out"]), dtype=self.torch_dtype, device="cuda")
        if state is None:
            conv_forward(self.plan, self.graph, schedule, x, pos, shift, phi, A, out, self.workspace(OP_FORWARD))
        else:
            conv_forward_keep_state(self.plan, self.graph, x, pos, shift, phi, A, out, state,
                                    self.workspace(OP_FORWARD))
        return out

    def backward(self, x, pos, shift, phi, A, grad_out, want=("x", "pos", "edge_vec", "phi", "A"), state=None):
        import torch
        n, e = self.graph.n_nodes, self.graph.n_edges
        info = self.plan.info
        dt = dict(dtype=self.torch_dtype, device="cuda")
        outs = dict(
            x=torch.empty((n, info["c_in"]), **dt) if "x" in want else None,
            pos=torch.empty((n, 3), **dt) if "pos" in want else None,
            edge_vec=torch.empty((max(e, 1), 3), **dt) if "edge_vec" in want else None,
            phi=torch.empty((max(e, 1), info["num_radial"]), **dt) if "phi" in want else None,
            A=torch.empty((info["num_radial"], info["n_weights"]), **dt) if "A" in want else None,
        )
        if state is None:
            conv_backward(self.plan, self.graph, x, pos, shift, phi, A, grad_out, grad_x=outs["x"],
                          grad_pos=outs["pos"], grad_edge_vec=outs["edge_vec"], grad_phi=outs["phi"],
                          grad_A=outs["A"], workspace=self.workspace(OP_BACKWARD))
        else:
            conv_backward_with_state(self.plan, self.graph, x, pos, shift, phi, A, grad_out, state,
                                     grad_x=outs["x"], grad_pos=outs["pos"], grad_edge_vec=outs["edge_vec"],
                                     grad_phi=outs["phi"], grad_A=outs["A"], workspace=self.workspace(OP_BACKWARD))
        return {k: v for k, v in outs.items() if v is not None}

    def triple_backward(self, inputs: dict, want=TRIPLE_OUTPUTS):
        """Third-order derivative on the edge operand Y (see conv_triple_backward); returns the
        requested outputs as new device tensors."""
        import torch
        n, e = self.graph.n_nodes, self.graph.n_edges
        info = self.plan.info
        dt = dict(dtype=self.torch_dtype, device="cuda")
        shapes = dict(x=(n, info["c_in"]), Y=(max(e, 1), info["sh_dim"]), phi=(max(e, 1), info["num_radial"]),
                      A=(info["num_radial"], info["n_weights"]), grad_out=(n, info["c_out"]))
        outs = {k: torch.empty(shapes[k.replace("v_", "")], **dt) for k in want}
        conv_triple_backward(self.plan, self.graph, inputs, outs, self.workspace(OP_TRIPLE_BACKWARD))
        return outs

    def double_backward(self, x, pos, shift, phi, A, grad_out, v_x=None, v_pos=None, v_edge_vec=None, v_phi=None,
                        v_A=None, want=("x", "pos", "edge_vec", "phi", "A", "grad_out")):
        """Gradients of <v, backward(x, r, phi, A, grad_out)> with respect to every backward input."""
        import torch
        n, e = self.graph.n_nodes, self.graph.n_edges
        info = self.plan.info
        dt = dict(dtype=self.torch_dtype, device="cuda")
        outs = dict(
            x=torch.empty((n, info["c_in"]), **dt) if "x" in want else None,
            pos=torch.empty((n, 3), **dt) if "pos" in want else None,
            edge_vec=torch.empty((max(e, 1), 3), **dt) if "edge_vec" in want else None,
            phi=torch.empty((max(e, 1), info["num_radial"]), **dt) if "phi" in want else None,
            A=torch.empty((info["num_radial"], info["n_weights"]), **dt) if "A" in want else None,
            grad_out=torch.empty((n, info["c_out"]), **dt) if "grad_out" in want else None,
        )
        conv_double_backward(self.plan, self.graph, x, pos, shift, phi, A, grad_out, v_x=v_x, v_pos=v_pos,
                             v_edge_vec=v_edge_vec, v_phi=v_phi, v_A=v_A, gg_x=outs["x"], gg_pos=outs["pos"],
                             gg_edge_vec=outs["edge_vec"], gg_phi=outs["phi"], gg_A=outs["A"],
                             gg_grad_out=outs["grad_out"], workspace=self.workspace(OP_DOUBLE_BACKWARD))
        return {k: v for k, v in outs.items() if v is not None}
