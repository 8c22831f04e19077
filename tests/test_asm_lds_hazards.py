"""The kernels' inline-asm LDS reads, checked in their own gfx950 assembly (CPU only).

The forward and backward kernels read LDS through inline asm (`ds_read_b128`,
`ds_read_b64_tr_b16`) and wait for the results with explicit `s_waitcnt lgkmcnt(N)`.
The compiler takes an asm output as written when the asm statement ends, so it may
copy, spill or reuse that register while the read is still in flight; only the
kernel's own waits keep that from happening.  This test compiles every .hip source to
device assembly with the library's flags and walks every kernel:

- an asm LDS read is complete once `lgkmcnt(N)` has been waited with at least N LDS
  reads issued after it (LDS reads return in order; other lgkm traffic only makes
  the wait stricter);
- no instruction may read or write a destination register of an asm LDS read that
  is not complete yet (that is the copy / spill / reuse hazard);
- no asm LDS read may still be in flight at a branch or a block label (the compiler
  can insert copies at block boundaries).

Reads the compiler emits itself (plain C++ loads from LDS) carry its own waits and
are not tracked.  A variant that held V fragments across the forward's overflow
check branch produced NaN outputs on the GPU; this check reports it (spills of
in-flight registers, reads in flight at the branch).
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

build = pytest.importorskip("flexible_mask_flash_amd.build")

_REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _kernels(text):
    lines = text.split("\n")
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", lines[i])
        if m:
            j = i + 1
            while j < len(lines) and not lines[j].startswith(".Lfunc_end"):
                j += 1
            yield m.group(1), lines[i + 1:j]
            i = j
        i += 1


def lds_asm_hazards(body):
    """Findings (line, message) of one kernel body."""
    findings, outstanding, in_asm = [], [], False
    for n, line in enumerate(body):
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        s = line.split(";")[0].strip()
        if not s:
            continue
        if re.match(r"^\.LBB\w+:", s) or s.startswith(("s_branch", "s_cbranch", "s_setpc", "s_endpgm")):
            if outstanding:
                findings.append((n, "asm LDS read in flight at a block boundary: " + s))
            outstanding = []
            continue
        if s.startswith("."):
            continue
        op = s.split()[0]
        args = s[len(op):]
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", args)
            if m:
                k = int(m.group(1))
                outstanding = outstanding[len(outstanding) - k:] if 0 < k < len(outstanding) else \
                    ([] if k == 0 else outstanding)
            continue
        used = _regs(args)
        for ln, dest in outstanding:
            if used & dest:
                findings.append((n, f"register of an asm LDS read (line {ln}) touched before its wait: {s}"))
        if in_asm and op.startswith(("ds_read", "ds_load")):
            outstanding.append((n, _regs(args.split(",")[0])))
    return findings


def test_checker_flags_a_read_used_before_its_wait():
    body = [";;#ASMSTART", "\tds_read_b128 v[8:11], v1 offset:0", ";;#ASMEND",
            "\tscratch_store_dwordx4 off, v[8:11], off", "\ts_waitcnt lgkmcnt(0)", "\ts_endpgm"]
    assert len(lds_asm_hazards(body)) == 1
    ok = [";;#ASMSTART", "\tds_read_b128 v[8:11], v1 offset:0", ";;#ASMEND",
          ";;#ASMSTART", "\tds_read_b128 v[12:15], v1 offset:16", ";;#ASMEND",
          ";;#ASMSTART", "\ts_waitcnt lgkmcnt(1)", ";;#ASMEND",
          "\tv_mov_b32 v0, v8", "\ts_waitcnt lgkmcnt(0)", "\tv_mov_b32 v0, v12", "\ts_endpgm"]
    assert lds_asm_hazards(ok) == []
    late = [";;#ASMSTART", "\tds_read_b128 v[8:11], v1 offset:0", ";;#ASMEND", "\ts_cbranch_vccz .LBB0_2"]
    assert len(lds_asm_hazards(late)) == 1


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    """{source: gfx950 assembly text} of every .hip source, built with the library's flags."""
    tmp = tmp_path_factory.mktemp("asm")
    srcs = [s for s in build.SOURCES if s.endswith(".hip")]
    outs = [str(tmp / (s + ".s")) for s in srcs]

    def run(cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]

    with ThreadPoolExecutor(max_workers=3) as ex:
        list(ex.map(run, [build.asm_command(s, o) for s, o in zip(srcs, outs)]))
    return {s: open(o).read() for s, o in zip(srcs, outs)}


def test_kernels_never_touch_an_asm_lds_read_before_its_wait(device_asm):
    n_kernels, bad = 0, []
    for src, text in device_asm.items():
        for name, body in _kernels(text):
            n_kernels += 1
            bad += [(src, name, f) for f in lds_asm_hazards(body)]
    assert n_kernels >= 40
    assert not bad, bad[:5]


def test_backward_main_kernels_are_split_between_the_two_objects(device_asm):
    """ffa_bwd.hip (max-ILP scheduler) holds the D = 64 and 128 instances of ffa_bwd_main
    and declares the D = 16 and 32 ones extern; ffa_bwd_small.hip compiles those.  Each of
    the 48 instances (4 head dims x 2 element types x dQ, dK/dV, total attention, each
    with and without the soft cap) must be in exactly one object, the one of its head dim."""
    def mains(src):
        names = [n for n, _ in _kernels(device_asm[src]) if "ffa_bwd_main" in n]
        return {n: int(re.search(r"ffa_bwd_mainILi(\d+)E", n).group(1)) for n in names}

    big, small = mains("ffa_bwd.hip"), mains("ffa_bwd_small.hip")
    assert sorted(set(big.values())) == [64, 128] and len(big) == 24
    assert sorted(set(small.values())) == [16, 32] and len(small) == 24
    assert not set(big) & set(small)
