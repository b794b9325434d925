"""Properties of the generated gfx950 code that the kernels' performance and
correctness rest on, checked on the CPU from hipcc's assembly output:

* no scratch (private) memory in any kernel -- an early version staged the
  key/value tiles through scratch and wrote ~40 GB per launch;
* the attention kernel fits two waves per SIMD (<= 256 VGPRs);
* no packed fp32 VALU instructions (v_pk_{add,mul,fma}_f32), which the build
  disables;
* in the attention kernel's key loop, the direct-to-LDS copy of the next tile
  is not waited for (vmcnt) before the current tile's LDS reads: the only
  vmcnt(0) waits sit right before the per-tile barrier;
* the wide attention kernel keeps its O accumulators in AGPRs through its
  whole key loop (no accvgpr copies there), waits for tile copies only at the
  per-tile barrier, and every MFMA it issues from inline asm has the two wait
  states an MFMA needs after VALU code wrote one of its A/B operands (the
  compiler does not insert them for inline asm);
* the same two wait states in the backward kernels, and in every bf16 kernel
  no instruction other than a chained MFMA reads an AGPR within 18 wait
  states of an MFMA writing it (the compiler cannot see that inline-asm MFMAs
  wrote the accumulators it copies; a missed case returned stale values for
  the last accumulator rows of the dK/dV tail);
* the backward's tile loops wait for copies only right before their barrier;
* no kernel moves registers by run-time index (s_set_gpr_idx / v_movrel): a
  loop the compiler declines to unroll fully indexes its register arrays
  that way, as the dK/dV loop over its 8 ring slots did past the default
  unrolling threshold.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    from attention_qk_rmsnorm_amd.build import CSRC, HIPCC_FLAGS, INCLUDE, sources
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = {}
    d = tmp_path_factory.mktemp("asm")
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    for src in sources():
        name = os.path.basename(src)
        dst = d / (name + ".s")
        subprocess.run([hipcc, *flags, "-S", "--cuda-device-only", "-I", INCLUDE, "-I", CSRC,
                        src, "-o", str(dst)], check=True, capture_output=True)
        out[name] = dst.read_text()
    return out


def _kernels(text):
    """(name, body) of every kernel in an assembly file."""
    parts = re.split(r"^(_Z\S+):\s*;", text, flags=re.M)
    return [(parts[i], parts[i + 1]) for i in range(1, len(parts) - 1, 2)]


def test_no_scratch_in_bf16_kernels(asm):
    # the fp32 debug kernels hold a whole head row per thread and may spill
    for name, text in asm.items():
        for kname, body in _kernels(text):
            if "f32" in kname:
                continue
            sizes = re.findall(r"; ScratchSize: (\d+)", body)
            assert sizes and all(int(x) == 0 for x in sizes), f"{kname} uses scratch: {sizes}"


def test_attention_two_waves_per_simd(asm):
    text = asm["attn_narrow.hip"]
    vgprs = [int(x) for x in re.findall(r"; NumVgprs: (\d+)", text)]
    assert vgprs and max(vgprs) <= 256, vgprs
    occ = [int(x) for x in re.findall(r"; Occupancy: (\d+)", text)]
    assert occ and min(occ) >= 2, occ


def test_no_packed_fp32_valu(asm):
    for name, text in asm.items():
        assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", text), name


def test_tile_copy_not_waited_before_reads(asm):
    text = asm["attn_narrow.hip"]
    lines = [l.strip() for l in text.splitlines()]
    lds_dma = [i for i, l in enumerate(lines) if l.startswith("global_load_lds_dwordx4")]
    assert lds_dma, "attention kernel copies tiles with global_load_lds_dwordx4"
    # the in-loop copies follow the per-tile barrier, which the loop takes
    # right after waiting for the current tile's copy (vmcnt(0)); after each
    # such group a vmcnt wait may only be the one right before the next
    # barrier, never one ahead of an LDS read.  (The Q rows' copy before the
    # loop may follow another barrier, and is waited for on purpose.)
    groups = [i for j, i in enumerate(lds_dma) if j + 1 == len(lds_dma) or lds_dma[j + 1] - i > 8]
    firsts = [i for j, i in enumerate(lds_dma) if j == 0 or i - lds_dma[j - 1] > 8]

    def after_tile_barrier(first):
        for k in range(first - 1, max(0, first - 48) - 1, -1):
            if lines[k].startswith("s_barrier"):
                return lines[k - 1].startswith("s_waitcnt") and "vmcnt(0)" in lines[k - 1]
        return False

    in_loop = [last for first, last in zip(firsts, groups) if after_tile_barrier(first)]
    assert len(in_loop) >= 2, "expected the tile copies of both loop halves"
    checked = 0
    for i in in_loop:
        pending_wait = None
        for l in lines[i + 1:]:
            if l.startswith("s_waitcnt") and "vmcnt" in l:
                pending_wait = l
            elif l.startswith("ds_read"):
                assert pending_wait is None, f"vmcnt wait before the tile's LDS reads: {pending_wait}"
                checked += 1
                break
            elif l.startswith("s_barrier") or l.startswith("s_endpgm"):
                break
    assert checked == len(in_loop)


def _kernel(text, marker):
    for name, body in _kernels(text):
        if marker in name:
            return body
    raise AssertionError(f"kernel {marker} not found")


def _main_loop(body):
    """Lines of the first loop with MFMAs in it: the blocks the compiler
    annotates as that loop's header or as lying in it (LLVM places latch
    blocks before the header, so the loop is not one contiguous range from the
    header to a branch back to it)."""
    lines = [l.strip() for l in body.splitlines()]
    blocks, cur = [], None
    for l in lines:
        m = re.match(r"^(?:\.L(BB\d+_\d+):|; %bb\.\d+:)(.*)$", l)
        if m:
            own = m.group(1)
            note = m.group(2)
            if "Loop Header" in note:
                hdr = own
            else:
                h = re.search(r"Header=(BB\d+_\d+)", note)
                hdr = h.group(1) if h else None
            cur = [hdr, own, []]
            blocks.append(cur)
        elif cur is not None:
            cur[2].append(l)
    headers = [b[1] for b in blocks if b[0] is not None and b[0] == b[1]]
    for h in headers:
        loop = [x for b in blocks if b[0] == h for x in b[2]]
        if any(x.startswith("v_mfma") for x in loop):
            return loop
    raise AssertionError("no loop with MFMAs")


def test_wide_kernel_registers(asm):
    text = asm["attn_wide.hip"]
    for key in ("NumVgprs", "NumAgprs"):
        vals = [int(x) for x in re.findall(rf"; {key}: (\d+)", text)]
        assert vals and max(vals) <= 256, (key, vals)
    # O (128) and the Q operands (64) live in AGPRs
    assert min(int(x) for x in re.findall(r"; NumAgprs: (\d+)", text)) >= 128


def test_wide_kernel_loop_keeps_accumulators_in_agprs(asm):
    loop = _main_loop(_kernel(asm["attn_wide.hip"], "wide_kernelILb0"))
    assert sum(l.startswith("v_mfma") for l in loop) >= 64
    moves = [l for l in loop if l.startswith("v_accvgpr_")]
    assert not moves, moves[:4]


def test_wide_kernel_waits_for_copies_only_at_barriers(asm):
    loop = _main_loop(_kernel(asm["attn_wide.hip"], "wide_kernelILb0"))
    code = [l for l in loop if l and not l.startswith(";")]
    waits = 0
    for i, l in enumerate(code):
        if l.startswith("s_waitcnt") and "vmcnt" in l:
            waits += 1
            # the next barrier comes before any LDS read or MFMA
            nxt = next((x for x in code[i + 1:]
                        if x.startswith(("s_barrier", "ds_read", "v_mfma"))), None)
            assert nxt is not None and nxt.startswith("s_barrier"), code[i:i + 6]
    assert waits >= 2


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


@pytest.mark.parametrize("source, minimum", [("attn_wide.hip", 100), ("bwd.hip", 40)])
def test_inline_asm_mfma_wait_states(asm, source, minimum):
    text = asm[source]
    lines = [l.strip() for l in text.splitlines()]
    inasm, checked, bad = False, 0, []
    for i, l in enumerate(lines):
        if l.startswith(";;#ASMSTART"):
            inasm = True
        elif l.startswith(";;#ASMEND"):
            inasm = False
        elif inasm and l.startswith("v_mfma"):
            checked += 1
            ops = [t.strip() for t in l.split(None, 1)[1].split(",")]
            srcs = _regs(ops[1]) | _regs(ops[2])
            slots, j = 0, i - 1
            while slots < 2 and j >= 0:
                p = lines[j]
                j -= 1
                if not p or p.startswith(";") or p.endswith(":"):
                    continue
                op = p.split()[0]
                if op == "s_nop":
                    slots += int(p.split()[1]) + 1
                    continue
                if op.startswith("v_") and not op.startswith("v_mfma"):
                    if _regs(p.split(None, 1)[1].split(",")[0].strip()) & srcs:
                        bad.append((p, l))
                slots += 1
    assert checked >= minimum
    assert not bad, bad[:3]


def _agpr_read_hazards(body):
    """(mfma, reader, wait states) where a non-MFMA instruction reads an AGPR
    that an MFMA wrote fewer than 18 wait states earlier (an MFMA issue is
    counted as 8 states, its pass count at most; labels end the search)."""
    lines = [l.split(";")[0].strip() for l in body.splitlines()]
    lines = [l for l in lines if l and not (l.startswith(".") and not l.endswith(":"))]
    found = []
    for i, l in enumerate(lines):
        if l.endswith(":") or l.startswith("v_mfma") or not l.startswith("v_") or " " not in l:
            continue
        srcs = set()
        for tok in l.split(None, 1)[1].split(",")[1:]:
            srcs |= {r for r in _regs(tok.strip()) if r[0] == "a"}
        if not srcs:
            continue
        gap = 0
        for p in reversed(lines[max(0, i - 40):i]):
            if p.endswith(":"):
                break
            if p.startswith("v_mfma"):
                if _regs(p.split(None, 1)[1].split(",")[0].strip()) & srcs and gap < 18:
                    found.append((p, l, gap))
                gap += 8
            elif p.startswith("s_nop"):
                gap += int(p.split()[1]) + 1
            else:
                gap += 1
    return found


def test_agpr_reads_wait_for_mfma_results(asm):
    for source in ("attn_narrow.hip", "attn_wide.hip", "bwd.hip"):
        for kname, body in _kernels(asm[source]):
            hz = _agpr_read_hazards(body)
            assert not hz, (kname[:60], hz[:3])


def test_backward_loops_wait_for_copies_only_at_barriers(asm):
    # after every group of tile copies, up to the next barrier in the code,
    # a vmcnt wait may only stand right before that barrier (the ring's own
    # wait): a wait between the copies and the step's LDS reads would drain
    # the copies just issued
    text = asm["bwd.hip"]
    # every instantiation: the dQ kernel's 8-wave form unrolls a ring of 4
    # key tiles, its 4-wave form a ring of 2
    cases = [(name, body) for name, body in _kernels(text)
             if "bwd_dkdv_kernel" in name or "bwd_dq_kernel" in name]
    assert len(cases) >= 6, [n for n, _ in cases]
    for marker, body in cases:
        minimum = 2 if "bwd_dq_kernel" in marker and "Li4E" in marker else 4
        code = [l.split(";")[0].strip() for l in body.splitlines()]
        code = [l for l in code if l and not l.startswith(".")]
        copies = [i for i, l in enumerate(code) if l.startswith("global_load_lds")]
        ends = [i for j, i in enumerate(copies) if j + 1 == len(copies) or copies[j + 1] - i > 12]
        checked = 0
        for end in ends:
            nxt = next((k for k in range(end + 1, len(code)) if "s_barrier" in code[k]), None)
            if nxt is None:
                continue
            reads = any(code[k].startswith("ds_read") for k in range(end + 1, nxt))
            if not reads:
                continue  # the ring prologue: its wait precedes its barrier anyway
            for k in range(end + 1, nxt):
                if code[k].startswith("s_waitcnt") and "vmcnt" in code[k]:
                    assert nxt - k <= 8, (marker, code[k], code[k + 1:k + 4])
            checked += 1
        assert checked >= minimum, (marker[:60], checked)


def test_no_indexed_register_moves(asm):
    for name, text in asm.items():
        for kname, body in _kernels(text):
            hits = re.findall(r"^\s*(s_set_gpr_idx_on|v_movrel\w*)", body, flags=re.M)
            assert not hits, (name, kname[:70], len(hits))
