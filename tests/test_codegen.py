"""Code-generation guards for the grouped GEMM (CPU only; needs hipcc).

The GEMM pipeline relies on properties of the gfx950 code the compiler emits:
  * the K loop must never drain every in-flight copy (no `s_waitcnt vmcnt(0)`
    in a block that issues MFMAs): each stage waits for its own copies with
    an exact count, and a full drain would serialise the multi-stage pipeline;
  * no GEMM variant may spill registers or use scratch memory.
Both have regressed silently before (a second LDS object made the compiler
drain the copies), so they are checked on the assembly of every variant.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routing_dispatch_expert_gate_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _compile(flags):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-fhip-fp32-correctly-rounded-divide-sqrt", "-x", "hip",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-c", os.path.join(CSRC, "ffn.hip"),
           "--cuda-device-only"] + flags
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return r


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "ffn.s"
    r = _compile(["-S", "-o", str(out), "-Rpass-analysis=kernel-resource-usage"])
    return out.read_text(), r.stderr


def _kernels(text):
    return re.findall(r"^(_ZN3moe12_GLOBAL__N_19gg_kernel\w+):", text, re.M)


def test_k_loop_never_drains_all_copies(asm):
    text, _ = asm
    names = _kernels(text)
    assert len(names) >= 20, names
    for name in names:
        a = text.index(name + ":")
        b = text.index(".Lfunc_end", a)
        for blk in re.split(r"\n(?=\.LBB)", text[a:b]):
            if "v_mfma" in blk:
                assert not re.search(r"s_waitcnt vmcnt\(0\)", blk), f"{name}: K-loop block drains vmcnt"


def test_gemm_variants_do_not_spill(asm):
    _, remarks = asm
    cur = None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            continue
        if cur and "gg_kernel" in cur:
            for key in ("VGPRs Spill", "ScratchSize [bytes/lane]"):
                m = re.search(re.escape(key) + r": (\d+)", line)
                if m:
                    assert int(m.group(1)) == 0, f"{cur}: {key} = {m.group(1)}"


@pytest.mark.parametrize("src", ["route.hip", "align.hip", "combine.hip"])
def test_small_kernels_use_no_scratch(src, tmp_path):
    """Route, align and combine kernels keep everything in registers and LDS:
    a device function left out of line (a call) spills to scratch."""
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-fhip-fp32-correctly-rounded-divide-sqrt", "-x", "hip",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "--cuda-device-only",
           "-o", str(tmp_path / "k.o"), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    cur = None
    seen = 0
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            seen += 1
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m:
            assert int(m.group(1)) == 0, f"{cur} uses scratch"
    assert seen > 0


def test_fused_router_loop_never_drains_all_copies(tmp_path):
    """The fused E <= 64 router streams Wg through LDS stages behind its x
    loads: inside the K loop each stage waits for its own copies only (the
    single LDS allocation keeps the compiler from draining them)."""
    out = tmp_path / "route.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-fhip-fp32-correctly-rounded-divide-sqrt", "-x", "hip",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-S", os.path.join(CSRC, "route.hip"),
           "--cuda-device-only", "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    text = out.read_text()
    names = re.findall(r"^(_ZN3moe12_GLOBAL__N_118route_fused_kernel\w+):", text, re.M)
    # six (parts, substeps) shapes, with and without codes, in 8- and 16-wave workgroups
    assert len(names) == 24, names
    for name in names:
        a = text.index(name + ":")
        b = text.index(".Lfunc_end", a)
        body = text[a:b]
        # the kernel's stage count S, from its template arguments as the kernel
        # derives it (<QUANT, KQ, NSUB, NW, LDSB>)
        kq, nsub, nw, ldsb = map(int, re.search(r"route_fused_kernelILb[01]ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E",
                                                name).groups())
        rb = 64 if kq >= 8 else 128
        nst = nsub // (rb // 64)
        smax = ldsb // (64 * kq * rb)
        stages = max(nst + 1, 2) if nst + 1 < smax else smax
        # the loop is unrolled: every wait from the first barrier to the last
        # MFMA, except the final stage's, leaves later copies in flight (before
        # the first barrier the codes variants publish the row maxima to LDS,
        # and the compiler drains the prefetched stages once for that write).
        # With two stages the copy in flight at a stage's wait is that stage's
        # own, so every wait is vmcnt(0) by design: there, no more than one
        # wait per stage.
        first = body.index("s_barrier")
        last = body.rindex("v_mfma")
        waits = re.findall(r"s_waitcnt vmcnt\((\d+)\)", body[first:last])
        if stages == 2:
            assert len(waits) <= nst, (name, waits)
        else:
            assert all(int(w) > 0 for w in waits[:-1]), (name, waits)
