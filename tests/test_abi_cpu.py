"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe.h declares, and its host-side validation returns the documented
status before any launch (every call here fails validation or has T == 0)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16, I8 = 0, 1, 2
P = ctypes.c_void_p(256)   # a non-null, aligned dummy pointer: never dereferenced on these paths


@pytest.fixture(scope="module")
def moe():
    lib_path = os.path.join(ROOT, "routing_dispatch_expert_gate_amd", "libmoe.so")
    if not os.path.exists(lib_path):
        import __graft_entry__
        __graft_entry__._build_module().build()
    import routing_dispatch_expert_gate_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_header_symbols_exported(moe):
    names = declared_functions()
    assert len(names) == 24, names
    for n in names:
        assert hasattr(moe.lib, n), n
        assert n in moe.SIGNATURES, n


def test_capacity_and_sizes(moe):
    L = moe.lib
    assert L.moe_capacity(4096, 8, 256, 1.25) == 160
    assert L.moe_capacity(16384, 6, 64, 1.25) == 1920
    assert L.moe_capacity(10, 3, 4, 1.25) == 10
    assert L.moe_capacity(64, 2, 8, 0.0) == 0
    assert L.moe_capacity(7, 1, 3, 1.1) == 3          # ceil(2.566..)
    # 1.1 * 80 * 2 / 16 is 11 for the decimal, a little above 11 for the double
    assert L.moe_capacity(80, 2, 16, 1.1) == 11
    assert L.moe_capacity(100, 1, 10, 1.1) == 11
    assert L.moe_capacity(10, 1, 1, 0.3) == 3        # 0.3 * 10: the double is just below
    assert L.moe_capacity(64, 2, 8, 1e-7) == -1      # outside [2^-20, 2^30]
    assert L.moe_capacity(64, 2, 8, 2.0 ** 31) == -1
    assert L.moe_align_max_tiles(4096, 2, 8, 128) == 64 + 8
    assert L.moe_align_max_tiles(16, 8, 256, 128) == 1 + 128
    assert L.moe_ffn_block_m(4096, 4096, 14336, 8, 2, BF16) in (16, 32, 64, 128, 256)
    assert L.moe_ffn_block_m(4096, 4096, 14336, 8, 2, 7) == -1
    small = L.moe_layer_workspace_size(64, 128, 256, 8, 2, F32, F32)
    big = L.moe_layer_workspace_size(4096, 4096, 14336, 8, 2, BF16, BF16)
    assert 0 < small < big
    assert big >= 4096 * 2 * 4096 * 2        # the expert-sorted output rows at least
    # partial logits [ks][T][E] fp32 (256-byte aligned), then per-split row absmax [ks][T]
    # large batch: 128 x 128 tiles, K split in 4 (partial logits and row absmax per split)
    assert L.moe_route_workspace_size(4096, 4096, 256, 8) == 4 * (4096 * 256 * 4 + 4096 * 4)
    assert L.moe_route_workspace_size(4096, 4096, 8, 2) == 0


def _route(moe, **kw):
    a = dict(x=P, xd=BF16, wg=P, wd=BF16, bias=None, T=64, H=128, E=8, k=2, ids=P, w=P, p=None,
             xq=None, xs=None, ws=None, nws=0)
    a.update(kw)
    return moe.lib.moe_route(a["x"], a["xd"], a["wg"], a["wd"], a["bias"], a["T"], a["H"], a["E"], a["k"],
                             a["ids"], a["w"], a["p"], a["xq"], a["xs"], a["ws"], a["nws"], None)


def test_route_validation(moe):
    msg = lambda: moe.lib.moe_last_error().decode()   # noqa: E731
    assert _route(moe, k=9, E=8) == INVALID and "k (9)" in msg()
    assert _route(moe, k=0) == INVALID
    assert _route(moe, T=-1) == INVALID
    assert _route(moe, E=300, k=2) == UNSUPPORTED
    assert _route(moe, E=16, k=9) == UNSUPPORTED           # k > 8
    assert _route(moe, H=100) == UNSUPPORTED
    assert _route(moe, E=24, k=2) == UNSUPPORTED           # E > 16 must be a multiple of 16
    assert _route(moe, E=64, wd=F32) == UNSUPPORTED        # E > 16 needs bf16 wg
    assert _route(moe, E=8, H=4096 * 4) == UNSUPPORTED     # beyond the register-resident slice
    assert _route(moe, x=None) == INVALID and "x" in msg()
    assert _route(moe, ids=None) == INVALID
    assert _route(moe, xq=P) == INVALID                    # xq without xs
    assert _route(moe, xd=I8) == UNSUPPORTED
    assert _route(moe, x=ctypes.c_void_p(258)) == INVALID  # misaligned
    assert _route(moe, E=256, k=8, H=512) == WORKSPACE     # logits workspace needed
    assert _route(moe, E=256, k=8, H=512, ws=ctypes.c_void_p(4096 + 8), nws=1 << 30) == WORKSPACE
    assert _route(moe, T=0) == OK
    assert moe.lib.moe_last_dispatch().decode() == "none (T=0)"


def test_route_grouped_validation(moe):
    L = moe.lib
    msg = lambda: L.moe_last_error().decode()   # noqa: E731

    def rg(T=64, H=512, E=256, k=8, G=8, TG=4, xd=BF16, wd=BF16, ws=None, nws=0):
        return L.moe_route_grouped(P, xd, P, wd, None, T, H, E, k, G, TG, P, P, None, None, None, ws, nws, None)

    assert rg(G=7) == INVALID and "n_group" in msg()       # does not divide E
    assert rg(G=128, E=256) == INVALID                    # more than 64 groups
    assert rg(TG=0) == INVALID
    assert rg(TG=9) == INVALID and "topk_group" in msg()
    assert rg(E=64, G=8, TG=1, k=9) == UNSUPPORTED        # k > 8 fails first
    assert rg(E=64, G=16, TG=1, k=6) == INVALID and "kept groups" in msg()
    assert rg(E=16, G=4, TG=2, k=2) == UNSUPPORTED        # E <= 16: no grouped path
    assert rg(wd=F32) == UNSUPPORTED
    assert rg() == WORKSPACE
    assert rg(T=0) == OK
    assert L.moe_route_workspace_size(64, 512, 256, 8) > 0


def test_route_align_validation(moe):
    L = moe.lib

    def ra(T=16, E=256, k=8, bm=64, H=512, o=P, ws=None, nws=0, wd=BF16):
        return L.moe_route_align(P, BF16, P, wd, None, T, H, E, k, 0, bm, P, P, None, None, None, o, o, o, o, o, o, o,
                                 ws, nws, None)

    assert ra(bm=100) == INVALID
    assert ra(o=None) == INVALID
    assert ra(k=9) == UNSUPPORTED
    assert ra(wd=F32) == UNSUPPORTED           # E > 16 needs bf16 wg
    assert ra() == WORKSPACE                   # the logits workspace
    assert ra(T=0) == OK
    assert L.moe_route_align_workspace_size(16, 512, 256, 8) >= L.moe_route_workspace_size(16, 512, 256, 8)
    assert L.moe_route_align_workspace_size(4096, 512, 8, 8) >= L.moe_align_workspace_size(4096, 8, 8) > 0


def test_pack_int4_and_w4a16_validation(moe):
    L = moe.lib
    assert L.moe_pack_int4(P, 4, 96, P, None) == UNSUPPORTED     # K % 64
    assert L.moe_pack_int4(P, -1, 64, P, None) == INVALID
    assert L.moe_pack_int4(None, 4, 64, P, None) == INVALID
    assert L.moe_pack_int4(P, 4, 64, ctypes.c_void_p(264), None) == INVALID   # misaligned
    assert L.moe_pack_int4(P, 0, 64, None, None) == OK
    I4 = 3
    assert L.moe_ffn_block_m(16, 4096, 1024, 256, 8, I4) == 64
    assert L.moe_ffn_block_m(4096, 4096, 1024, 8, 2, I4) == 256
    # W4A16 needs bf16 activations and both scale arrays
    n = L.moe_ffn_workspace_size(64, 256, 128, 8, 2, I4)
    assert n >= 64 * 2 * 128 * 2
    bm = L.moe_ffn_block_m(64, 256, 128, 8, 2, I4)

    def ffn(act=BF16, s13=P, s2=P, T=64):
        return L.moe_expert_ffn(P, act, None, P, P, I4, s13, s2, P, P, P, bm, None, T, 256, 128, 8, 2, P, BF16,
                                None, 0, None)

    assert ffn(act=F32) == UNSUPPORTED
    assert ffn(act=I8) == UNSUPPORTED
    assert ffn(s13=None) == INVALID
    assert ffn(s2=None) == INVALID
    assert ffn() == WORKSPACE
    assert ffn(T=0) == OK

    def layer(xd=BF16, s=P):
        return L.moe_layer(P, xd, P, BF16, None, P, P, I4, s, s, 64, 256, 128, 8, 2, 0, P, xd, None, None, 0, None)

    assert layer(xd=F32) == UNSUPPORTED
    assert layer(s=None) == INVALID
    assert layer() == WORKSPACE


def test_align_validation(moe):
    L = moe.lib

    def call(**kw):
        a = dict(ids=P, T=64, k=2, E=8, C=0, bm=128, out=P, ws=None, nws=0)
        a.update(kw)
        o = a["out"]
        return L.moe_align(a["ids"], a["T"], a["k"], a["E"], a["C"], a["bm"], o, o, o, o, o, o, o,
                           a["ws"], a["nws"], None)

    assert call(bm=100) == INVALID
    assert call(k=3, E=2) == INVALID
    assert call(ids=None) == INVALID
    assert call(out=None) == INVALID
    # above 2^14 slots the three-launch path needs its histogram workspace;
    # at or below it one workgroup needs none
    assert call(T=2049, k=8) == WORKSPACE
    assert L.moe_align_workspace_size(2049, 8, 8) > 0
    assert L.moe_align_workspace_size(2048, 8, 8) == 0
    assert call(T=0) == OK


def test_ffn_validation(moe):
    L = moe.lib

    def call(ad=BF16, wd=BF16, yd=BF16, bm=None, T=64, H=128, I=128, E=8, k=2, xs=None, s=None, ws=None, nws=0):
        if bm is None:
            bm = L.moe_ffn_block_m(T, H, I, E, k, wd)
        return L.moe_expert_ffn(P, ad, xs, P, P, wd, s, s, P, P, P, bm, None, T, H, I, E, k, P, yd, ws, nws,
                                None)

    assert call(ad=F32, wd=BF16) == UNSUPPORTED
    assert call(yd=F32) == UNSUPPORTED
    assert call(I=96) == UNSUPPORTED
    assert call(ad=I8, wd=I8, H=192, xs=P, s=P) == UNSUPPORTED     # W8A8 needs multiples of 128
    assert call(ad=I8, wd=I8, xs=None, s=P) == INVALID
    assert call(bm=64 if L.moe_ffn_block_m(64, 128, 128, 8, 2, BF16) != 64 else 32) == INVALID
    assert call() == WORKSPACE
    assert call(T=0) == OK


def test_combine_and_layer_validation(moe):
    L = moe.lib
    assert L.moe_combine(P, I8, P, None, 64, 2, 128, P, BF16, None) == UNSUPPORTED
    assert L.moe_combine(None, BF16, P, None, 64, 2, 128, P, BF16, None) == INVALID
    assert L.moe_combine(P, BF16, P, None, 0, 2, 128, P, BF16, None) == OK

    def cs(T=64, shared=None, f=1.0, bias=None, out=P, yd=BF16, od=BF16, H=128):
        return L.moe_combine_shared(P, yd, P, None, T, 2, H, shared, f, bias, out, od, None)

    assert cs(yd=I8) == UNSUPPORTED
    assert cs(H=96) == UNSUPPORTED
    assert cs(f=float("nan")) == INVALID
    assert cs(f=float("inf"), T=0) == INVALID          # the factor is checked even for T == 0
    assert cs(out=None) == INVALID
    assert cs(bias=ctypes.c_void_p(260)) == INVALID    # bias must be 16-byte aligned
    assert cs(shared=ctypes.c_void_p(272)) == INVALID  # overlaps out without being out
    assert cs(T=0) == OK

    def layer(xd=BF16, wd=BF16, od=BF16, T=64, H=128, I=128, E=8, k=2, ws=None, nws=0, s=None):
        return L.moe_layer(P, xd, P, BF16, None, P, P, wd, s, s, T, H, I, E, k, 0, P, od, None, ws, nws, None)

    assert layer(od=F32) == UNSUPPORTED
    assert layer(xd=F32, wd=BF16, od=F32) == UNSUPPORTED
    assert layer(wd=I8) == INVALID                     # scales missing
    assert layer() == WORKSPACE
    assert layer(T=0) == OK


def test_layer_options_validation(moe):
    """moe_layer_ex checks its options before anything is enqueued."""
    L = moe.lib

    def ex(ng=0, tg=0, shared=None, f=1.0, ob=None, T=64, E=32, k=2, opts=True):
        o = moe.binding.MoeLayerOptions(ng, tg, shared, f, ob)
        return L.moe_layer_ex(P, BF16, P, BF16, None, P, P, BF16, None, None, T, 128, 128, E, k, 0, P, BF16,
                              None, ctypes.byref(o) if opts else None, None, 0, None)

    assert ex(opts=False) == WORKSPACE               # NULL options: moe_layer
    assert ex() == WORKSPACE
    assert ex(ng=4, tg=2) == WORKSPACE
    assert ex(ng=3, tg=1) == INVALID                 # n_group must divide E
    assert ex(ng=4, tg=5) == INVALID                 # topk_group > n_group
    assert ex(ng=8, tg=1, k=5) == INVALID            # k above the kept groups' experts
    assert ex(ng=2, tg=1, E=8) == UNSUPPORTED        # group-limited routing needs 16 < E <= 256
    assert ex(f=float("nan")) == INVALID
    assert ex(f=float("inf"), T=0) == INVALID        # checked even for T == 0
    assert ex(ob=ctypes.c_void_p(260)) == INVALID    # out_bias must be 16-byte aligned
    assert ex(shared=ctypes.c_void_p(272)) == INVALID  # overlaps out without being out
    assert ex(shared=P) == WORKSPACE                 # shared may be out itself
    assert ex(T=0, ng=4, tg=2) == OK


def test_mfma_probe_is_outside_the_library(moe):
    """The bench's MFMA-rate probe lives in its own library, not in the
    library's ABI; its argument errors return before any launch."""
    assert not hasattr(moe.lib, "moe_probe_mfma_rate")
    probe = ctypes.CDLL(os.path.join(ROOT, "routing_dispatch_expert_gate_amd", "libmoe_probe.so"))
    f = probe.moe_probe_mfma_rate
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert f(0, 10, ctypes.c_void_p(256), None) == -1
    assert f(4, 0, ctypes.c_void_p(256), None) == -1
    assert f(4, 10, None, None) == -1


def test_capacity_equals_oracle_over_a_grid(moe):
    """moe_capacity takes the factor as the same bounded-denominator fraction
    as the oracle (reading R1), over decimal and random factors and loads
    whose quotient is or is not an integer."""
    import numpy as np

    import oracle
    L = moe.lib
    rng = np.random.default_rng(3)
    factors = [0.1, 0.2, 0.3, 0.7, 0.9, 1.0, 1.05, 1.1, 1.15, 1.2, 1.25, 1.3, 1.35, 1.5, 1.7, 1.9, 2.0, 2.2,
               2.5, 3.3, 4.4, 1 / 3, 2 / 3, 1 / 7, 0.001, 0.000123, 123.456, 1000.5, 2.0 ** -20, 2.0 ** 30]
    factors += [round(float(f), int(d)) for f, d in zip(rng.uniform(0.01, 20, 60), rng.integers(1, 7, 60))]
    factors += rng.uniform(0.01, 50, 40).tolist()
    loads = [(1, 1, 1), (7, 1, 3), (10, 3, 4), (80, 2, 16), (100, 1, 10), (333, 2, 8), (4096, 8, 256),
             (16384, 6, 64), (1000, 5, 7), (2 ** 20 + 3, 8, 256), (50, 8, 10), (12345, 4, 100)]
    for f in factors:
        for T, k, E in loads:
            want = oracle.capacity(T, k, E, f)
            assert L.moe_capacity(T, k, E, f) == want, (T, k, E, f, want)


def test_binding_structs_match_the_header(moe, tmp_path):
    """The ctypes mirrors of the header's structs (moe_layer_aux,
    moe_layer_options) have the header's size and member offsets, as a C
    compiler lays them out."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"moe_layer_aux": moe.binding.MoeLayerAux, "moe_layer_options": moe.binding.MoeLayerOptions}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "moe.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    r = subprocess.run([cc, "-std=c11", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            cname, what, val = line.split()
            got[(cname, what)] = int(val)
    for cname, py in structs.items():
        assert got[(cname, "sizeof")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
