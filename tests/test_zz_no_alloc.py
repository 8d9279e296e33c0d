"""moe_layer_noalloc (the allocation-free layer) against moe_layer, called
through the C ABI: two calls in a row on the library's own scratch array,
the second with a smaller batch, each bit-identical to moe_layer with a
caller workspace on the same inputs; a shape beyond the scratch is refused
before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import moe_synth

pytestmark = pytest.mark.gpu


def _dev(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class _Inputs:
    def __init__(self, spec, seed):
        import routing_dispatch_expert_gate_amd as moe
        i = moe_synth.make_inputs(spec, seed)
        self.spec = spec
        self.x, self.wg, self.bias = _dev(i.x), _dev(i.wg), _dev(i.bias)
        self.w13, self.w2, self.s13, self.s2 = _dev(i.w13), _dev(i.w2), _dev(i.s13), _dev(i.s2)
        self.wdt = {"bf16": moe.MOE_BF16, "i8": moe.MOE_I8, "i4a8": moe.MOE_I4A8, "f32": moe.MOE_F32}[spec.w_dtype]
        if spec.w_dtype == "i4a8":
            self.w13, self.w2 = moe.pack_int4(self.w13), moe.pack_int4(self.w2)
        self.C = moe.capacity(spec.T, spec.k, spec.E, spec.capacity_factor) if spec.capacity_factor > 0 else 0


def _call(d, noalloc, out, ids, pos):
    import routing_dispatch_expert_gate_amd as moe
    L = moe.lib
    s = d.spec
    DT = moe.binding._DT
    st = moe.binding._stream(d.x.device)
    aux = moe.binding.MoeLayerAux(topk_ids=ids.data_ptr(), pos=pos.data_ptr())
    args = (_p(d.x), DT[d.x.dtype], _p(d.wg), DT[d.wg.dtype], _p(d.bias), _p(d.w13), _p(d.w2), d.wdt, _p(d.s13),
            _p(d.s2), s.T, s.H, s.I, s.E, s.k, d.C, _p(out), DT[out.dtype], ctypes.byref(aux))
    if noalloc:
        return L.moe_layer_noalloc(*args, st)
    n = int(L.moe_layer_workspace_size(s.T, s.H, s.I, s.E, s.k, DT[d.x.dtype], d.wdt))
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    rc = L.moe_layer(*args, _p(ws), n, st)
    torch.cuda.synchronize()
    return rc


def _run_both(spec, seed):
    import routing_dispatch_expert_gate_amd as moe
    d = _Inputs(spec, seed)
    s = spec
    outs = {}
    for noalloc in (True, False):
        out = torch.full((s.T, s.H), 7.0, dtype=d.x.dtype, device="cuda")
        ids = torch.full((s.T, s.k), -5, dtype=torch.int32, device="cuda")
        pos = torch.full((s.T, s.k), -5, dtype=torch.int32, device="cuda")
        rc = _call(d, noalloc, out, ids, pos)
        torch.cuda.synchronize()
        assert rc == 0, moe.lib.moe_last_error().decode()
        if noalloc:
            assert "no-alloc scratch" in moe.last_dispatch()
        outs[noalloc] = (out, ids, pos)
    a, b = outs[True], outs[False]
    for u, v in zip(a, b):
        if u.dtype == torch.bfloat16:
            u, v = u.view(torch.int16), v.view(torch.int16)
        assert torch.equal(u, v)
    return a[0]


def test_noalloc_layer_equals_layer_twice_second_smaller():
    import routing_dispatch_expert_gate_amd as moe
    print("[noalloc] decode-sized bf16, E=256, T=64 (capacity), then W8A8 T=16", flush=True)
    big = moe_synth.Spec("na_bf16_T64_E256_cap", 64, 1024, 256, 8, 256, capacity_factor=1.25)
    small = moe_synth.Spec("na_w8a8_T16_E64", 16, 512, 64, 6, 256, w_dtype="i8", zipf_s=1.1)
    o1 = _run_both(big, 11)
    o2 = _run_both(small, 12)
    assert o1.abs().max().item() > 0 and o2.abs().max().item() > 0
    # the first workload again, after the smaller one left its scratch behind
    _run_both(big, 11)
    # the decode workload of the pages' fine-grained router (W4A8 weights)
    _run_both(moe_synth.CONFIGS[4].replace(name="na_decode_w4a8", w_dtype="i4a8"), 13)
    print(f"[noalloc] ok: {moe.last_dispatch()}", flush=True)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    import routing_dispatch_expert_gate_amd as moe
    L = moe.lib
    T, H, I, E, k = 4096, 4096, 14336, 8, 2
    need = int(L.moe_layer_workspace_size(T, H, I, E, k, moe.MOE_BF16, moe.MOE_BF16))
    assert need > 16 << 20
    P = ctypes.c_void_p(256)
    rc = L.moe_layer_noalloc(P, moe.MOE_BF16, P, moe.MOE_BF16, None, P, P, moe.MOE_BF16, None, None, T, H, I, E, k, 0,
                             P, moe.MOE_BF16, None, None)
    assert rc == moe.binding.MOE_ERR_UNSUPPORTED
    assert "scratch" in L.moe_last_error().decode()
    # T == 0 is a no-op, as for moe_layer
    assert L.moe_layer_noalloc(None, moe.MOE_BF16, None, moe.MOE_BF16, None, P, P, moe.MOE_BF16, None, None, 0, H,
                               I, E, k, 0, P, moe.MOE_BF16, None, None) == 0
