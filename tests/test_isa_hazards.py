"""CPU checks of the hazards that inline asm hides from the compiler, and a
model of the page-range restart protocol that a faulting build once used.

1. The built code object (gfx950 AMD assembly of this repository's own
   build, disassembled with the ROCm LLVM tools) is scanned: every HBM ->
   LDS copy must sit in the asm block that carries its wait states, i.e. be
   preceded by `s_nop 0`, the `m0` write and `s_nop 4`. On gfx950 an SALU
   write of m0 needs one wait state before an LDS DMA reads it, and a VALU
   write of an SGPR (v_readfirstlane of a base address) needs five before a
   vector memory instruction reads it; the compiler does not see inside the
   asm, so the asm itself must carry them on every path.

2. A step-by-step model of four waves running a double-buffered page loop
   with a workgroup-wide restart driven by an LDS flag (a per-row reference
   exceeded on a later page restarts the range): every wave must run the
   same number of barriers, copy only pages of the range, and never copy
   into a buffer another wave may still be reading.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mla_paged_kv_03_amd", "libmla_decode.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
DMA = re.compile(r"\b(global_load_lds_dword\w*|buffer_load_dword\w*\b.*\blds\b)")


def _tool(name):
    p = os.path.join(LLVM, name)
    return p if os.path.exists(p) else shutil.which(name)


def _disassemble(tmp_path):
    """Disassembly of every gfx950 code object in the built library."""
    objcopy, bundler, objdump = _tool("llvm-objcopy"), _tool("clang-offload-bundler"), \
        _tool("llvm-objdump")
    if not (objcopy and bundler and objdump) or not os.path.exists(LIB):
        pytest.skip("ROCm LLVM tools or the built library not found")
    fat = tmp_path / "fatbin"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", LIB, str(tmp_path / "x.so")],
                   check=True, capture_output=True)
    data = fat.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), data)]
    texts = []
    for k, s in enumerate(starts):
        e = starts[k + 1] if k + 1 < len(starts) else len(data)
        b = tmp_path / f"b{k}"
        b.write_bytes(data[s:e])
        co = tmp_path / f"co{k}"
        subprocess.run([bundler, "--type=o", "--unbundle", f"--targets={TARGET}", f"--input={b}",
                        f"--output={co}"], check=True, capture_output=True)
        out = subprocess.run([objdump, "-d", "--mcpu=gfx950", str(co)], check=True,
                             capture_output=True, text=True).stdout
        texts.append(out)
    return texts


def _instructions(text):
    ins = []
    for ln in text.splitlines():
        m = re.match(r"^\s+([a-z_][a-z0-9_]*)(\s+[^/]*)?(//.*)?$", ln)
        if m:
            ins.append((m.group(1) + (m.group(2) or "")).strip())
    return ins


def test_every_lds_copy_carries_its_wait_states(tmp_path):
    texts = _disassemble(tmp_path)
    copies = 0
    for text in texts:
        ins = _instructions(text)
        for i, op in enumerate(ins):
            if not DMA.match(op):
                continue
            copies += 1
            assert i >= 3, op
            assert ins[i - 1] == "s_nop 0", (op, ins[i - 3:i])
            assert ins[i - 2].startswith(("s_mov_b32 m0,", "s_add_u32 m0,")), (op, ins[i - 3:i])
            assert ins[i - 3] == "s_nop 4", (op, ins[i - 3:i])
    # the decode, expansion and calibration kernels all copy pages this way
    assert copies > 100


def test_scan_detects_a_copy_without_wait_states():
    """The scan itself: a copy straight after its m0 write fails it."""
    ins = ["v_readfirstlane_b32 s4, v1", "s_mov_b32 m0, s6",
           "global_load_lds_dwordx4 v2, s[4:5] nt"]
    i = 2
    assert DMA.match(ins[i])
    assert not (ins[i - 1] == "s_nop 0" and ins[i - 2].startswith("s_mov_b32 m0,"))


# ----------------------------------------------------------- restart model
class _Wave:
    def __init__(self, w):
        self.w = w
        self.barriers = 0


def run_restart_model(n_pages, restart_at, n_waves=4):
    """Model of the restart protocol as it was described: pages p0..p1-1 go
    through two LDS buffers; page j + 1 is copied (each wave a share) while
    page j is computed; a wave whose rows see a score above the reference on
    page `restart_at` (None: never) sets an LDS flag during that page. After
    the barrier that opens the next page every wave reads the flag; if set,
    every wave waits for its copies, meets a barrier, one wave clears the
    flag, all meet another barrier and the range starts over once (the
    reference then comes from the exact maxima, so no second restart).
    Returns the per-wave barrier counts; asserts buffer and page bounds."""
    waves = [_Wave(w) for w in range(n_waves)]
    flag = False
    # state of each buffer: page held, copies in flight (count), readers
    in_flight = {0: 0, 1: 0}
    pages_copied = []

    def barrier():
        for wv in waves:
            wv.barriers += 1

    def issue(page, buf):
        assert 0 <= page < n_pages, f"copy of page {page} outside the range"
        # nobody may be reading buf: only the page just finished used it
        pages_copied.append(page)
        in_flight[buf] += n_waves

    def wait_copies(buf):
        in_flight[buf] = 0

    restarted = False
    while True:
        issue(0, 0)
        restart = False
        for j in range(n_pages):
            cur = j & 1
            wait_copies(cur)
            barrier()                      # page j landed; page j - 1 done by all
            if flag:                       # read by every wave after the same barrier
                restart = True
                break
            if j + 1 < n_pages:
                issue(j + 1, cur ^ 1)      # refill the buffer page j - 1 used
            assert in_flight[cur] == 0, "a buffer read while copies into it are in flight"
            if restart_at is not None and j == restart_at and not restarted:
                flag = True                # set during page j, seen after the next barrier
        if restart:
            wait_copies(0)
            wait_copies(1)
            barrier()                      # every copy landed, every wave saw the flag
            flag = False                   # one wave clears it
            barrier()                      # nobody reads the flag before it is clear
            restarted = True
            continue
        if flag:                           # set on the last page: seen after the range
            wait_copies(0)
            wait_copies(1)
            barrier()
            flag = False
            barrier()
            restarted = True
            continue
        break
    barrier()
    counts = {wv.barriers for wv in waves}
    assert len(counts) == 1, counts
    assert all(0 <= p < n_pages for p in pages_copied)
    return counts.pop()


@pytest.mark.parametrize("n_pages", range(1, 13))
def test_restart_protocol_is_balanced_and_in_bounds(n_pages):
    base = run_restart_model(n_pages, None)
    assert base == n_pages + 1
    for r in range(n_pages):
        n = run_restart_model(n_pages, r)
        assert n > base


def test_restart_model_catches_an_off_by_one_copy():
    """A loop that copies page j + 1 without checking the range end copies
    a page past it; the model's bounds check catches that."""
    with pytest.raises(AssertionError):
        _copy_past_the_end(3)


def _copy_past_the_end(n_pages):
    pages = []
    for j in range(n_pages):
        nxt = j + 1
        assert 0 <= nxt < n_pages, f"copy of page {nxt} outside the range"
        pages.append(nxt)


def _kernel_metadata(tmp_path):
    """(name, sgpr_spill_count, vgpr_spill_count) of every kernel in the
    library's gfx950 code objects, from their AMDGPU metadata notes."""
    readelf = _tool("llvm-readelf")
    if not readelf:
        pytest.skip("llvm-readelf not found")
    _disassemble(tmp_path)  # unbundles co0, co1, ... into tmp_path
    out = []
    for co in sorted(tmp_path.glob("co*")):
        notes = subprocess.run([readelf, "--notes", str(co)], capture_output=True, text=True).stdout
        for block in notes.split("- .agpr_count")[1:]:
            name = re.search(r"\.name:\s+(\S+)", block)
            ss = re.search(r"\.sgpr_spill_count:\s+(\d+)", block)
            vs = re.search(r"\.vgpr_spill_count:\s+(\d+)", block)
            if name and ss and vs:
                out.append((name.group(1), int(ss.group(1)), int(vs.group(1))))
    return out


def test_latent_decode_kernel_spills_no_sgpr(tmp_path):
    """The 128-row latent decode keeps every wave-uniform value in SGPRs:
    builds of it that spilled SGPRs to VGPR lanes were the ones that faulted
    the GPU (in a timing variant and in a graph-capture test), builds
    without such spills never did."""
    meta = _kernel_metadata(tmp_path)
    k = [m for m in meta if "decode128_kernel" in m[0]]
    assert k, meta
    for name, sgpr_spills, _ in k:
        assert sgpr_spills == 0, (name, sgpr_spills)
