"""The row-broadcast FMAs of the channelwise kernels (v_fmac_f32_dpp and v_mul_f32_dpp with
row_newbcast) and the in-row transposing adds of their per-edge channel reductions (v_add_f32_dpp
with row_mirror, row_half_mirror and quad permutations under bank masks) are inline assembly,
whose operand hazards the compiler does not check: on gfx9 a DPP instruction must not read a VGPR
that a VALU instruction wrote fewer than two wait states before.  The generated kernels feed the
broadcasts only registers filled by memory loads and start every group of reduction adds with
two wait states; this test compiles 16-, 32- and 64-channel plans (forward, backward, double
backward: four, two and one edge per wave) and a fully connected plan, and checks every DPP
instruction in the disassembled code objects, following branches into each instruction's
predecessors.  Runs on the CPU (the compiler targets gfx950 without a GPU)."""
import os
import re
import shutil
import subprocess

import pytest

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

_INST = re.compile(r"^\s+(\S+)(.*?)//\s*([0-9A-Fa-f]+):")
_TARGET = re.compile(r"<(\S+)\+0x([0-9a-fA-F]+)>")
_FUNC = re.compile(r"^([0-9a-fA-F]+) <(\S+)>:")


def _vregs(tok):
    tok = tok.strip()
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _parse(text):
    """Instructions as (address, opcode, operands) plus the function start addresses."""
    insts, funcs = [], {}
    for line in text.splitlines():
        f = _FUNC.match(line)
        if f:
            funcs[f.group(2)] = int(f.group(1), 16)
            continue
        m = _INST.match(line)
        if m:
            insts.append((int(m.group(3), 16), m.group(1), m.group(2).strip()))
    return insts, funcs


def _hazards(text):
    insts, funcs = _parse(text)
    index = {a: k for k, (a, _, _) in enumerate(insts)}
    preds = {k: [] for k in range(len(insts))}
    for k, (a, op, args) in enumerate(insts):
        if op.startswith("s_cbranch") or op == "s_branch":
            t = _TARGET.search(args)
            if t and t.group(1) in funcs:
                dst = funcs[t.group(1)] + int(t.group(2), 16)
                if dst in index:
                    preds[index[dst]].append(k)
        if k + 1 < len(insts) and op not in ("s_branch", "s_endpgm", "s_setpc_b64"):
            preds[k + 1].append(k)

    def writes(k, regs):
        _, op, args = insts[k]
        if not op.startswith("v_") or op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
            return False
        return bool(_vregs(args.split(",")[0]) & regs)

    def wait_states(k):
        _, op, args = insts[k]
        if op == "s_nop":
            return int(args.split()[0], 0) + 1
        return 1

    bad, count = [], 0
    for k, (a, op, args) in enumerate(insts):
        if not op.endswith("_dpp"):
            continue
        count += "row_newbcast" in args
        src0 = _vregs(args.split(",")[1])
        # depth-first over predecessors until two wait states separate them from the DPP read
        stack = [(j, 0) for j in preds[k]]
        seen = set()
        while stack:
            j, ws = stack.pop()
            if (j, ws) in seen:
                continue
            seen.add((j, ws))
            if writes(j, src0):
                bad.append(f"{insts[j][1]} {insts[j][2]} -> {op} {args} at {a:#x}")
                break
            ws += wait_states(j)
            if ws < 2:
                stack.extend((i, ws) for i in preds[j])
    return count, bad


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="llvm-objdump not installed")
def test_row_broadcast_operands_come_from_loads(tmp_path, monkeypatch):
    import clebsch_gordan_tensor_receiver_amd as cg

    cache = tmp_path / "kernels"
    cache.mkdir()
    monkeypatch.setenv("CGTP_KERNEL_CACHE", str(cache))
    for c in (16, 32, 64):
        irreps = f"{c}x0e+{c}x1o+{c}x2e"
        plan = cg.Plan(irreps, "1x0e+1x1o+1x2e", irreps, "uvu", "float32", 8)
        plan.compile((0, 1, 2))
    cg.Plan("32x0e+32x1o", "1x0e+1x1o", "32x0e+32x1o", "uvw", "float32", 8).compile((0, 1))
    total = 0
    for co in sorted(cache.glob("*.co")):
        text = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(co)], check=True, capture_output=True,
                              text=True).stdout
        count, bad = _hazards(text)
        assert not bad, f"{co.name}: DPP source written by VALU within two wait states: {bad[:3]}"
        total += count
    # the forward, both backward passes and the double backward of these plans use the broadcast
    assert total > 1000
    shutil.rmtree(cache)


def test_hazard_scanner_flags_a_planted_hazard():
    """The scanner itself: a VALU write of the broadcast source right before the DPP read (no wait
    states) is flagged, one s_nop 1 in between clears it, and a write reaching the DPP through a
    branch is found too."""
    body = (
        "0000000000001000 <k>:\n"
        "\tv_mov_b32_e32 v5, 0 // 000000001000: 00000000\n"
        "\tv_fmac_f32_dpp v1, v5, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf // 000000001004: 00000000\n"
    )
    assert len(_hazards(body)[1]) == 1
    clear = body.replace("\tv_fmac", "\ts_nop 1 // 000000001002: 00000000\n\tv_fmac")
    assert _hazards(clear) == (1, [])
    branched = (
        "0000000000001000 <k>:\n"
        "\tv_mov_b32_e32 v5, 0 // 000000001000: 00000000\n"
        "\ts_branch 4 <k+0x10> // 000000001004: 00000000\n"
        "\ts_nop 7 // 000000001008: 00000000\n"
        "\ts_nop 7 // 00000000100C: 00000000\n"
        "\tv_fmac_f32_dpp v1, v5, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf // 000000001010: 00000000\n"
    )
    assert len(_hazards(branched)[1]) == 1
    # any DPP source, not only row broadcasts: the transposing adds of the reductions
    mirror = body.replace("v_fmac_f32_dpp v1, v5, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf",
                          "v_add_f32_dpp v1, v5, v5 row_mirror row_mask:0xf bank_mask:0xc")
    assert _hazards(mirror) == (0, ["v_mov_b32_e32 v5, 0 -> v_add_f32_dpp v1, v5, v5 row_mirror row_mask:0xf"
                                    " bank_mask:0xc at 0x1004"])
