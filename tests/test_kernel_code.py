"""Invariants of the generated gfx950 code of the FP8 attention kernels (CPU only:
hipcc cross-compiles the sources to assembly).

* Every tile / descale load that writes LDS directly is inline assembly that
  the compiler's hazard checks do not see; each must carry its own wait states
  (s_nop 4) so that a descriptor SGPR written by a VALU instruction, or M0, is
  never read stale.
* The unrolled main loop waits for its loads with a fixed vmcnt that counts
  only those loads, so it must contain no vector-memory operation of the
  compiler's own (scratch spills, global / flat accesses, buffer stores);
  scalar loads are counted separately (lgkmcnt) and are allowed.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "fp8_attention_forward_amd", "csrc", "attn_fp8.hip")
DECODE_SRC = os.path.join(ROOT, "fp8_attention_forward_amd", "csrc", "attn_decode.hip")
BF16_SRC = os.path.join(ROOT, "fp8_attention_forward_amd", "csrc", "attn_bf16.hip")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


_ASM = {}


def _assembly(src):
    if src not in _ASM:
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "--cuda-device-only", "-S", src, "-o", "-"]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert res.returncode == 0, res.stderr[-2000:]
        _ASM[src] = res.stdout
    return _ASM[src]


def _compile(src, pattern):
    parts = re.split(r"\n(?=_ZN7attnfp8(?:" + pattern + r")\S*:)", _assembly(src))
    funcs = {}
    for p in parts[1:]:
        name = p.split(":", 1)[0]
        funcs[name] = p.split("\n.Lfunc_end", 1)[0].splitlines()
    return funcs


def _resources(src, names):
    """Scratch bytes and waves per SIMD the compiler reports for each kernel."""
    asm = _assembly(src)
    out = {}
    for name in names:
        m = re.search(r"\.size\s+" + re.escape(name) + r",.*?; ScratchSize: (\d+).*?; Occupancy: (\d+)", asm, re.S)
        assert m, name
        out[name] = (int(m.group(1)), int(m.group(2)))
    return out


@pytest.fixture(scope="module")
def kernels():
    funcs = _compile(SRC, "15attn_fp8_kernel|22attn_fp8_varlen_kernel")
    # (dense, packed) x D x scale block x causal x exponential mode x MX, plus
    # the dense kernels with 32-channel MX scales (D x scale block x causal x
    # exponential mode)
    assert len(funcs) == 80, sorted(funcs)
    return funcs


def test_attention_kernels_run_three_waves_per_simd_without_spills(kernels):
    # the loop holds one score tile and reads K operands per subtile so that it
    # fits in 168 VGPRs: three waves per SIMD (LDS: 48 KiB per workgroup, three
    # workgroups per CU); a spill would also put compiler memory operations
    # into the loop that waits with a partial vmcnt
    for name, (scratch, occ) in _resources(SRC, kernels).items():
        assert scratch == 0, f"{name}: {scratch} bytes of scratch"
        assert occ >= 3, f"{name}: {occ} waves per SIMD"


@pytest.fixture(scope="module")
def decode_kernels():
    funcs = _compile(DECODE_SRC, "22attn_fp8_decode_kernel|31attn_fp8_decode_balanced_kernel")
    assert len(funcs) == 16, sorted(funcs)   # (fixed ranges, balanced shares) x D x scale block x causal
    return funcs


def _code(lines):
    return [l.strip() for l in lines if l.strip() and not l.strip().startswith(";")]


@pytest.fixture(scope="module")
def bf16_kernels():
    funcs = _compile(BF16_SRC, "16attn_bf16_kernel")
    assert len(funcs) == 4, sorted(funcs)   # D x causal
    return funcs


def test_bf16_kernels_run_three_waves_per_simd_without_spills(bf16_kernels):
    # 48 KiB of LDS per workgroup at D = 128 (two three-slot rings of 8 KiB
    # tiles): three workgroups per CU, so three waves per SIMD must fit the
    # registers too, and without scratch (a spill would be a vector-memory
    # operation inside loops that wait with a partial vmcnt)
    for name, (scratch, occ) in _resources(BF16_SRC, bf16_kernels).items():
        assert scratch == 0, f"{name}: {scratch} bytes of scratch"
        assert occ >= 3, f"{name}: {occ} waves per SIMD"


def test_every_lds_dma_carries_its_wait_states(kernels, decode_kernels, bf16_kernels):
    for name, lines in list(kernels.items()) + list(decode_kernels.items()) + list(bf16_kernels.items()):
        code = _code(lines)
        n = 0
        for i, ins in enumerate(code):
            if re.match(r"buffer_load_dword\S*\s.*\blds\b", ins):
                n += 1
                assert code[i - 1] == "s_nop 4", f"{name}: LDS DMA without its own wait states: {ins}"
        assert n > 0, name


def _loops(lines):
    """(label, body lines) of every loop: its header block, every block the
    compiler annotates as inside it ("in Loop: Header=..."; loops entered by
    fall-through have no branch to their header, so the annotations are the
    reliable record), and the bodies of the loops nested in it (whose headers
    say "Parent Loop ...")."""
    starts = [i for i, l in enumerate(lines) if re.match(r"^\.LBB\S+:", l)]
    blocks = []
    for k, st in enumerate(starts):
        end = starts[k + 1] if k + 1 < len(starts) else len(lines)
        head = lines[st] + (" " + lines[st + 1] if st + 1 < end and lines[st + 1].strip().startswith(";") else "")
        blocks.append((lines[st].split(":", 1)[0], st, end, head))
    hdr_of = lambda lab: lab[1:].replace("LBB", "BB", 1)   # annotations name .LBB0_13 as BB0_13

    def body_of(lab):
        hdr = hdr_of(lab)
        body = []
        for lab2, st2, end2, head2 in blocks:
            if lab2 == lab or re.search(r"in Loop: Header=" + re.escape(hdr) + r"\b", head2):
                body += lines[st2:end2]
            elif "Loop Header" in head2 and re.search(r"Parent Loop " + re.escape(hdr) + r"\b", head2):
                body += body_of(lab2)
        return body

    return [(lab, body_of(lab)) for lab, st, end, head in blocks if "Loop Header" in head]


def _asm_blocks(lines):
    """Instructions written as inline assembly (between the ASMSTART/ASMEND markers)."""
    out, inside = [], False
    for l in lines:
        if "ASMSTART" in l:
            inside = True
        elif "ASMEND" in l:
            inside = False
        elif inside and l.strip():
            out.append(l.strip())
    return out


def test_partial_tile_waits_count_only_tile_loads(kernels, bf16_kernels):
    """A loop that waits for its tile loads with a partial vmcnt (the kernel's
    own inline s_waitcnt) must not contain vector-memory operations of the
    compiler's own, which that count does not include."""
    for name, lines in list(kernels.items()) + list(bf16_kernels.items()):
        n_partial = 0
        for lab, body in _loops(lines):
            mine = [w for w in _asm_blocks(body) if re.match(r"s_waitcnt vmcnt\((\d+)\)", w)]
            if not any(int(re.search(r"\d+", w).group()) > 0 for w in mine):
                continue
            n_partial += 1
            mem = [l.strip() for l in body if re.search(r"\b(scratch_|global_|flat_|buffer_store)", l)]
            assert not mem, f"{name} {lab}: compiler vector-memory operations in a loop with partial waits: {mem[:4]}"
        assert n_partial >= 1, name   # the main loop keeps loads in flight across steps


def test_decode_waits_for_its_tile_loads_in_full(decode_kernels):
    """The decode loop's V tiles arrive by LDS DMA that the compiler does not
    count: every loop that issues them (the tile loop, and in the balanced
    kernels the loop over pieces around it) must wait with a full vmcnt(0)
    (seen by the compiler) and keep no partial wait of its own, and no decode
    kernel may spill."""
    for name, lines in decode_kernels.items():
        loops = [(lab, body) for lab, body in _loops(lines)
                 if any(re.match(r"buffer_load_dword\S*\s.*\blds\b", l.strip()) for l in body)]
        assert len(loops) == (2 if "balanced" in name else 1), name
        # the tile loop (the innermost): only full waits; the loop over pieces
        # around it may hold the compiler's own partial waits for its own
        # loads (the queries of the next piece), which untracked loads can
        # only make longer
        _, tile_loop = min(loops, key=lambda lb: len(lb[1]))
        waits = [l.strip() for l in tile_loop if l.strip().startswith("s_waitcnt") and "vmcnt" in l]
        assert waits and all("vmcnt(0)" in w for w in waits), f"{name}: {waits}"
        for _, body in loops:
            assert not _asm_blocks(body) or all(not w.startswith("s_waitcnt") for w in _asm_blocks(body))
    for name, (scratch, occ) in _resources(DECODE_SRC, decode_kernels).items():
        assert scratch == 0, f"{name}: {scratch} bytes of scratch"
        assert occ >= 2, f"{name}: {occ} waves per SIMD"
