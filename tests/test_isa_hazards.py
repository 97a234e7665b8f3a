"""gfx950 ISA of every kernel in the library: no MFMA result is read at the
start of a basic block sooner than that MFMA's required wait states after it
ends a predecessor block.

Within a block the compiler pads such reads itself; at a block start reached
by a branch it has been seen to omit that padding (a k-loop whose exit edge
led straight to the LDS write of the accumulators), which gives wrong
results in scattered tiles with no error.  The scan compiles each source
with the library's own flags (hipcc cross-compiles for gfx950 without a GPU)
and checks every block start against each predecessor's trailing MFMAs.
The scanner itself is pinned on two hand-written snippets."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from tensor_dit_transformer_amd import build as B

# Wait states an MFMA result needs before a vector-ALU, LDS or memory
# instruction may read it: passes + 3 for these (gfx950 bf16: 16x16x32 is
# 4 passes, 32x32x16 is 8 -- 16 and 32 cycles at the dense bf16 rate; fp32
# 32x32x2 is 16 passes, 64 cycles at the fp32 matrix rate); the compiler's
# own padding for the 16x16x32 accumulator read is 7.  An MFMA missing here
# fails the scan so that it gets an entry.
NEED_WAIT_STATES = {
    "v_mfma_f32_16x16x32_bf16": 7,
    "v_mfma_f32_32x32x16_bf16": 11,
    "v_mfma_f32_32x32x2_f32": 19,
}
LOOKBACK = 24   # beyond every entry above

pytestmark = pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC),
                                reason="hipcc not available")


def _regs(tok):
    m = re.match(r"([av])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([av])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _functions(text):
    funcs, cur = [], None
    for line in text.splitlines():
        s = line.split(";")[0].rstrip()
        if re.match(r"^_Z\w+:$", s):
            cur = {"name": s[:-1], "ins": []}
            funcs.append(cur)
            continue
        if cur is None:
            continue
        if s.startswith(".Lfunc_end"):
            cur = None
            continue
        m = re.match(r"^(\.LBB\w+):", s)
        if m:
            cur["ins"].append(("LABEL", m.group(1), []))
            continue
        s = s.strip()
        if not s or s.startswith("."):
            continue
        op = s.split()[0]
        rest = s[len(op):].strip()
        cur["ins"].append((op, rest, [o.strip() for o in rest.split(",")] if rest else []))
    return funcs


def _wait_states(op, rest):
    return int(rest.split()[0]) + 1 if op == "s_nop" else 1


def _reads(op, ops):
    if op.startswith(("ds_write", "global_store", "buffer_store", "flat_store")):
        return ops
    if op.startswith("v_mfma"):
        return ops[1:3]          # an accumulator chained as srcC is forwarded
    return ops[1:]


def scan(text):
    """(function, label, instruction, wait states) for every block-start read
    of an MFMA result sooner than that MFMA's NEED_WAIT_STATES after it ends
    a predecessor block."""
    found = []
    for f in _functions(text):
        ins = f["ins"]
        labels = {x[1]: i for i, x in enumerate(ins) if x[0] == "LABEL"}
        preds = {name: [] for name in labels}
        for i, (op, rest, _ops) in enumerate(ins):
            if op.startswith("s_cbranch") or op == "s_branch":
                target = rest.split()[0]
                if target in preds:
                    preds[target].append(i)
            if op == "LABEL" and i > 0 and ins[i - 1][0] != "s_branch":
                preds[rest].append(i - 1)
        for name, at in labels.items():
            for p in preds[name]:
                pending, dist, j = {}, 0, p
                while j >= 0 and dist < LOOKBACK and ins[j][0] != "LABEL":
                    op, rest, ops = ins[j]
                    if op.startswith("v_mfma") and ops:
                        if op not in NEED_WAIT_STATES:
                            found.append((f["name"], name, f"{op}: no wait-state entry", -1))
                        for r in _regs(ops[0]):
                            pending.setdefault(r, (dist, NEED_WAIT_STATES.get(op, LOOKBACK)))
                    dist += _wait_states(op, rest)
                    j -= 1
                if not pending:
                    continue
                elapsed = 0
                for k in range(at + 1, min(at + 16, len(ins))):
                    op, rest, ops = ins[k]
                    if op == "LABEL":
                        break
                    hit = [pending[r] for o in _reads(op, ops) for r in _regs(o) if r in pending]
                    if hit:
                        short = [(elapsed + d, need) for d, need in hit if elapsed + d < need]
                        if short:
                            found.append((f["name"], name, f"{op} {rest}", min(w for w, _ in short)))
                        break
                    elapsed += _wait_states(op, rest)
    return found


# A 4-pass MFMA, then a block reached by a branch (1 wait state) or by the
# fall-through past one s_nop (2), whose first instruction stores the result.
SNIPPET = """_Zk:
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]
\ts_cbranch_scc1 .LBB0_2
\ts_nop 0
.LBB0_2:
{pad}\tds_write_b128 v10, a[0:3]
\ts_endpgm
.Lfunc_end0:
"""


def test_scanner_flags_an_unpadded_block_start():
    hits = scan(SNIPPET.format(pad=""))
    # both ways in (the branch and the fall-through past one s_nop) are short
    assert [h[1] for h in hits] == [".LBB0_2", ".LBB0_2"]
    assert sorted(h[3] for h in hits) == [1, 2]


def test_scanner_accepts_a_padded_block_start():
    assert scan(SNIPPET.format(pad="\ts_nop 5\n")) == []          # 6 + 1 or 2 >= 7
    assert len(scan(SNIPPET.format(pad="\ts_nop 4\n"))) == 1      # 5 + 1 < 7 <= 5 + 2


def _device_isa(src, out):
    flags = [f for f in B.CFLAGS if f not in ("-fPIC", "-fvisibility=hidden")]
    cmd = [B.HIPCC, *flags, *B.FILE_FLAGS.get(os.path.basename(src), []), "--cuda-device-only",
           "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc -S failed on {src}:\n{r.stderr[-2000:]}"
    with open(out) as fh:
        return fh.read()


def test_no_mfma_result_read_too_early_at_a_block_start(tmp_path):
    srcs = B.sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        texts = list(ex.map(lambda s: _device_isa(s, str(tmp_path / (os.path.basename(s) + ".s"))), srcs))
    found = [(os.path.basename(s), h) for s, t in zip(srcs, texts) for h in scan(t)]
    assert sum(t.count("v_mfma") for t in texts) > 0, "no MFMA found: the scan read nothing"
    assert not found, "\n".join(f"{s}: {h}" for s, h in found)


# ---------------------------------------------------------------------------
# MFMAs issued from inline asm (the 64-query attention pins its accumulators
# to AGPRs that way) are not MFMAs to the compiler's hazard recognizer, so
# within a block it pads nothing around them.  The kernel's own fences, or
# the distance its schedule puts between an MFMA and the first use of its
# result, supply the wait states; this scan checks every such MFMA: on every
# path from it, through branches taken or not (a loop's back edge included),
# no instruction touches its result registers sooner than NEED_WAIT_STATES
# after it (a chained srcC of the next MFMA is forwarded by the hardware),
# and in straight-line code no vector instruction writes one of its source
# registers fewer than 2 wait states before it.
VALU_WRITE_TO_MFMA = 2


def _asm_blocks(text):
    """Per function, the instruction list with a flag for inline-asm lines."""
    funcs, cur, in_asm = [], None, False
    for line in text.splitlines():
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        s = line.split(";")[0].rstrip()
        if re.match(r"^_Z\w+:$", s):
            cur = []
            funcs.append((s[:-1], cur))
            continue
        if cur is None:
            continue
        if s.startswith(".Lfunc_end"):
            cur = None
            continue
        m = re.match(r"^(\.LBB\w+):", s)
        if m:
            cur.append(("LABEL", m.group(1), [], False))
            continue
        s = s.strip()
        if not s or s.startswith("."):
            continue
        for part in s.split("\n"):
            op = part.split()[0]
            rest = part[len(op):].strip()
            cur.append((op, rest, [o.strip() for o in rest.split(",")] if rest else [], in_asm))
    return funcs


def _touches_result(op2, ops2, dst):
    touched = set().union(*[_regs(o) for o in (ops2[1:3] if op2.startswith("v_mfma") else ops2)])
    if op2.startswith("v_mfma") and _regs(ops2[0]) == dst and dst <= set().union(*[_regs(o) for o in ops2[3:4]]):
        return False   # the next MFMA chaining the accumulator
    return bool(dst & touched)


def scan_inline_mfma(text):
    found = []
    for name, ins in _asm_blocks(text):
        labels = {x[1]: i for i, x in enumerate(ins) if x[0] == "LABEL"}
        for i, (op, rest, ops, asm) in enumerate(ins):
            if not (asm and op.startswith("v_mfma")):
                continue
            need = NEED_WAIT_STATES.get(op, LOOKBACK)
            dst = _regs(ops[0])
            srcs = set().union(*[_regs(o) for o in ops[1:4]])
            # later instructions touching the result, on every path (a branch
            # taken or not) until NEED_WAIT_STATES have passed
            paths, seen, hit = [(i + 1, 0)], set(), None
            while paths and hit is None:
                j, ws = paths.pop()
                if (j, ws) in seen:
                    continue
                seen.add((j, ws))
                while j < len(ins) and ws < need:
                    op2, rest2, ops2, _ = ins[j]
                    if op2 == "LABEL":
                        j += 1
                        continue
                    if op2 == "s_endpgm":
                        break
                    if op2 == "s_nop":
                        ws += int(rest2.split()[0]) + 1
                        j += 1
                        continue
                    if ops2 and _touches_result(op2, ops2, dst):
                        hit = (name, f"{op} {rest}", f"{op2} {rest2}", ws)
                        break
                    if op2.startswith(("s_cbranch", "s_branch")):
                        target = rest2.split()[0] if rest2 else ""
                        if target in labels:
                            paths.append((labels[target] + 1, ws + 1))
                        if op2 == "s_branch":
                            break
                    ws += 1
                    j += 1
            if hit:
                found.append(hit)
            # earlier vector writes of its sources
            ws = 0
            for j in range(i - 1, -1, -1):
                op2, rest2, ops2, _ = ins[j]
                if op2 == "LABEL" or ws >= VALU_WRITE_TO_MFMA:
                    break
                if op2 == "s_nop":
                    ws += int(rest2.split()[0]) + 1
                    continue
                if op2.startswith("v_") and not op2.startswith("v_mfma") and ops2 and _regs(ops2[0]) & srcs:
                    found.append((name, f"{op} {rest}", f"{op2} {rest2}", ws))
                    break
                ws += 1
    return found


INLINE_SNIPPET = """_Zk:
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
\t;;#ASMEND
{pad}\tv_accvgpr_read_b32 v10, a3
\tv_mov_b32_e32 v4, v10
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 a[16:31], v[0:3], v[4:7], a[16:31]
\t;;#ASMEND
\ts_endpgm
.Lfunc_end0:
"""


def test_inline_scanner_flags_unpadded_neighbours():
    hits = scan_inline_mfma(INLINE_SNIPPET.format(pad=""))
    # the accumulator read right after the first MFMA, the operand write right
    # before the second
    assert [h[2].split()[0] for h in hits] == ["v_accvgpr_read_b32", "v_mov_b32_e32"]


def test_inline_scanner_accepts_padding():
    hits = scan_inline_mfma(INLINE_SNIPPET.format(pad="\ts_nop 7\n\ts_nop 2\n"))
    assert [h[2].split()[0] for h in hits] == ["v_mov_b32_e32"]   # 11 wait states clear the read


# An MFMA whose result is read after a taken branch, at the top of a loop:
# only the path through the branch is short.
BRANCH_SNIPPET = """_Zk:
.LBB0_1:
{pad}\tv_accvgpr_read_b32 v10, a3
\ts_nop 7
\ts_nop 7
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
\t;;#ASMEND
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
.Lfunc_end0:
"""


def test_inline_scanner_follows_a_taken_branch():
    hits = scan_inline_mfma(BRANCH_SNIPPET.format(pad=""))
    assert [(h[2].split()[0], h[3]) for h in hits] == [("v_accvgpr_read_b32", 1)]
    # 1 (the branch) + 10 wait states clear it
    assert scan_inline_mfma(BRANCH_SNIPPET.format(pad="\ts_nop 9\n")) == []
    assert len(scan_inline_mfma(BRANCH_SNIPPET.format(pad="\ts_nop 8\n"))) == 1


def test_inline_asm_mfmas_are_padded(tmp_path):
    srcs = B.sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        texts = list(ex.map(lambda s: _device_isa(s, str(tmp_path / (os.path.basename(s) + ".s"))), srcs))
    n_inline = sum(len([1 for _, ins in _asm_blocks(t) for x in ins if x[3] and x[0].startswith("v_mfma")])
                   for t in texts)
    assert n_inline > 0, "no inline-asm MFMA found: the scan read nothing"
    found = [(os.path.basename(s), h) for s, t in zip(srcs, texts) for h in scan_inline_mfma(t)]
    assert not found, "\n".join(f"{s}: {h}" for s, h in found)
