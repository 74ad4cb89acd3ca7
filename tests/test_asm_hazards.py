"""Wait-state check of the inline-assembly MFMAs in the compiled main kernels.

The compiler inserts the wait states that the CDNA hazard rules require around the
instructions it generates, but not around inline assembly. The main kernel issues its
MFMAs (v_mfma_f32_32x32x16_bf16, 8 passes on gfx950) as inline assembly, so this test
compiles every (d, nw) variant with the library's own flags and walks the control-flow
graph of the generated assembly around each of them:
  - before: no VALU instruction may write an MFMA source register (A, B or C) less than
    2 wait states before the MFMA;
  - after: no other instruction may read or write the MFMA's result registers less than
    13 wait states after it, except a following MFMA that accumulates into exactly the
    same registers (srcC == vdst), which the hardware forwards.
A wait state is one instruction, or N + 1 for s_nop N. Paths are followed through
fall-through edges and through every branch to a label.
"""
import os
import re
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), ".."))

from scheduling_fa_attn_amd import build as dash_build  # noqa: E402

BEFORE = 2
AFTER = 13

_REG = re.compile(r"^([va])\[(\d+):(\d+)\]$|^([va])(\d+)$")


def _regs(tok):
    m = _REG.match(tok.strip())
    if not m:
        return frozenset()
    if m.group(1):
        return frozenset((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return frozenset({(m.group(4), int(m.group(5)))})


def _operands(text):
    parts = text.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip() for o in parts[1].split(",")]


class Inst:
    def __init__(self, text, asm):
        self.text = text
        self.op = text.split()[0]
        self.asm = asm  # inside an inline-assembly block
        ops = _operands(text)
        self.all_regs = frozenset().union(*[_regs(o) for o in ops]) if ops else frozenset()
        self.dst = _regs(ops[0]) if ops else frozenset()
        self.mfma = self.op.startswith("v_mfma")
        self.valu = self.op.startswith("v_") and not self.mfma
        if self.mfma:
            self.srcs = [_regs(o) for o in ops[1:4]]

    def wait_states(self):
        if self.op == "s_nop":
            return int(self.text.split()[1], 0) + 1
        return 1


def parse_kernel(asm_text, symbol):
    """Instructions and label positions of one kernel's function body."""
    insts, labels = [], {}
    inside = in_asm = False
    for raw in asm_text.splitlines():
        line = raw.split(";", 1)[0].strip() if not raw.strip().startswith(";;#ASM") else raw.strip()
        if raw.startswith(symbol + ":"):
            inside = True
            continue
        if not inside:
            continue
        if line == ";;#ASMSTART":
            in_asm = True
            continue
        if line == ";;#ASMEND":
            in_asm = False
            continue
        if line.startswith(".Lfunc_end"):
            break
        if line.endswith(":"):
            labels[line[:-1]] = len(insts)
            continue
        if not line or line.startswith("."):
            continue
        insts.append(Inst(line, in_asm))
    assert inside, f"kernel {symbol} not found"
    return insts, labels


def _succ_preds(insts, labels):
    n = len(insts)
    succ = [[] for _ in range(n)]
    for i, ins in enumerate(insts):
        op = ins.op
        if op.startswith("s_cbranch") or op == "s_branch":
            tgt = _operands(ins.text)[0] if _operands(ins.text) else ins.text.split()[1]
            assert tgt in labels, ins.text
            succ[i].append(labels[tgt])
        if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < n:
            succ[i].append(i + 1)
    preds = [[] for _ in range(n)]
    for i, ss in enumerate(succ):
        for s in ss:
            preds[s].append(i)
    return succ, preds


def find_hazards(insts, labels):
    succ, preds = _succ_preds(insts, labels)
    found = []
    for k, ins in enumerate(insts):
        if not (ins.mfma and ins.asm):
            continue
        srcs = frozenset().union(*ins.srcs)
        # Backward: VALU writes of a source register within BEFORE wait states.
        stack = [(p, 0) for p in preds[k]]
        seen = set()
        while stack:
            j, used = stack.pop()
            if (j, used) in seen:
                continue
            seen.add((j, used))
            p = insts[j]
            if p.valu and p.dst & srcs:
                found.append(f"{p.text}  ->  {ins.text}")
                continue
            used += p.wait_states()
            if used < BEFORE:
                stack.extend((q, used) for q in preds[j])
        # Forward: any access to the result registers within AFTER wait states.
        stack = [(s, 0) for s in succ[k]]
        seen = set()
        while stack:
            j, used = stack.pop()
            if (j, used) in seen:
                continue
            seen.add((j, used))
            p = insts[j]
            if p.all_regs & ins.dst:
                chained = p.mfma and p.srcs[2] == ins.dst and p.dst == ins.dst and not (
                    (p.srcs[0] | p.srcs[1]) & ins.dst)
                if not chained:
                    found.append(f"{ins.text}  ->  {p.text}")
                    continue
                # A chained MFMA's own result is checked from that MFMA.
                continue
            used += p.wait_states()
            if used < AFTER:
                stack.extend((q, used) for q in succ[j])
    return found


# Library flavours that run on the GPU: release, profiling (-DDASH_PROFILE), replay
# (-DDASH_REPLAY).
FLAVOURS = {"release": [], "profile": ["-DDASH_PROFILE"], "replay": ["-DDASH_REPLAY"]}


def _compile_asm(d, nw, flavour, out):
    cmd = [dash_build.HIPCC] + dash_build.COMMON + [f"-DDASH_MAIN_D={d}", f"-DDASH_MAIN_NW={nw}"] + \
        dash_build.MAIN_FLAGS[(d, nw)] + FLAVOURS[flavour] + \
        ["--cuda-device-only", "-S", "-x", "hip", os.path.join(dash_build.HERE, "csrc", "bwd_main.hip"), "-o", out]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    if not os.path.exists(dash_build.HIPCC):
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("asm")
    procs = {}
    for (d, nw) in dash_build.MAIN_FLAGS:
        for flavour in FLAVOURS:
            out = str(tmp / f"bwd_main_d{d}_nw{nw}_{flavour}.s")
            procs[(d, nw, flavour)] = (out, _compile_asm(d, nw, flavour, out))
    texts = {}
    for key, (out, proc) in procs.items():
        _, err = proc.communicate(timeout=600)
        assert proc.returncode == 0, err
        with open(out) as f:
            texts[key] = f.read()
    return texts


# (ordered reduction, cross-XCD chains, no dQ, per-tile partials): the five instantiations
# of each (d, nw), in every flavour.
VARIANTS = [(d, nw, det, cross, nodq, part, fl) for (d, nw) in sorted(dash_build.MAIN_FLAGS)
            for det, cross, nodq, part in ((1, 0, 0, 0), (1, 1, 0, 0), (0, 0, 0, 0), (0, 0, 1, 0), (1, 0, 0, 1))
            for fl in FLAVOURS]


@pytest.mark.parametrize("d,nw,det,cross,nodq,part,flavour", VARIANTS,
                         ids=[f"d{v[0]}-nw{v[1]}-det{v[2]}-cross{v[3]}-nodq{v[4]}-part{v[5]}-{v[6]}" for v in VARIANTS])
def test_inline_mfma_wait_states(kernel_asm, d, nw, det, cross, nodq, part, flavour):
    symbol = f"_ZN4dash15bwd_main_kernelILi{d}ELi{nw}ELb{det}ELb{cross}ELb{nodq}ELb{part}EEEvNS_9BwdParamsE"
    insts, labels = parse_kernel(kernel_asm[(d, nw, flavour)], symbol)
    n_mfma = sum(1 for i in insts if i.mfma and i.asm)
    assert n_mfma >= (32 if nodq else 48), n_mfma
    hazards = find_hazards(insts, labels)
    assert not hazards, "\n".join(hazards[:20])


def _compile_pair_asm(flavour, out):
    cmd = [dash_build.HIPCC] + dash_build.COMMON + dash_build.PAIR_FLAGS + FLAVOURS[flavour] + \
        ["--cuda-device-only", "-S", "-x", "hip", os.path.join(dash_build.HERE, "csrc", "bwd_pair.hip"), "-o", out]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


@pytest.fixture(scope="module")
def pair_asm(tmp_path_factory):
    if not os.path.exists(dash_build.HIPCC):
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("pair_asm")
    procs = {fl: (str(tmp / f"bwd_pair_{fl}.s"), None) for fl in FLAVOURS}
    procs = {fl: (out, _compile_pair_asm(fl, out)) for fl, (out, _) in procs.items()}
    texts = {}
    for fl, (out, proc) in procs.items():
        _, err = proc.communicate(timeout=600)
        assert proc.returncode == 0, err
        with open(out) as f:
            texts[fl] = f.read()
    return texts


# The two-waves-per-SIMD kernel (d = 128 and 64): ordered (fp32 final sums, or bf16 dQ
# written by the last contributors), atomic and per-tile partials instantiations, every
# flavour.
PAIR_VARIANTS = [(d, det, part, fused, fl) for d in (128, 64)
                 for det, part, fused in ((1, 0, 0), (1, 0, 1), (0, 0, 0), (1, 1, 0)) for fl in FLAVOURS]


@pytest.mark.parametrize("d,det,part,fused,flavour", PAIR_VARIANTS,
                         ids=[f"pair-d{v[0]}-det{v[1]}-part{v[2]}-fused{v[3]}-{v[4]}" for v in PAIR_VARIANTS])
def test_pair_kernel_inline_mfma_wait_states(pair_asm, d, det, part, fused, flavour):
    symbol = f"_ZN4dash15bwd_pair_kernelILi{d}ELb{det}ELb{part}ELb{fused}EEEvNS_9BwdParamsE"
    insts, labels = parse_kernel(pair_asm[flavour], symbol)
    # Both roles' bodies, d = 128: 16 + 16 + 8 per step and 8 for an item's last dQ block,
    # each; d = 64: 8 + 8 + 8 (A), 8 + 8 (B), and 8.
    n_mfma = sum(1 for i in insts if i.mfma and i.asm)
    assert n_mfma >= (96 if d == 128 else 48), n_mfma
    hazards = find_hazards(insts, labels)
    assert not hazards, "\n".join(hazards[:20])


def _synthetic(lines):
    text = "k:\n" + "\n".join(lines) + "\n.Lfunc_end0:\n"
    return parse_kernel(text, "k")


def test_checker_flags_planted_hazards():
    """The walk finds a VALU write right before an MFMA, one reached through a branch, and
    an early read of a result; it accepts the padded and chained forms."""
    mfma = ["\t;;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]", "\t;;#ASMEND"]
    ok = ["\tv_mov_b32 v17, 0", "\ts_nop 1"] + mfma + ["\ts_nop 7", "\ts_nop 4", "\tv_add_f32 v20, v0, v1"]
    assert find_hazards(*_synthetic(ok)) == []
    near = ["\tv_mov_b32 v17, 0", "\ts_nop 0"] + mfma
    assert len(find_hazards(*_synthetic(near))) == 1
    via_branch = ["\tv_mov_b32 v18, 0", "\ts_branch .LBB0_1", "\ts_nop 7", ".LBB0_1:"] + mfma
    assert len(find_hazards(*_synthetic(via_branch))) == 1
    early_read = ["\ts_nop 1"] + mfma + ["\ts_nop 7", "\tglobal_store_dwordx4 v[30:31], v[4:7], off"]
    assert len(find_hazards(*_synthetic(early_read))) == 1
    chained = ["\ts_nop 1"] + mfma + mfma + ["\ts_nop 15"]
    assert find_hazards(*_synthetic(chained)) == []
