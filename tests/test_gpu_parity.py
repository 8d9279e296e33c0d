"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (per workload):
  * top-k ids identical, except rows whose oracle k-th/(k+1)-th probability gap
    is below 1e-4 (counted and printed) and swaps of selected experts whose
    oracle probabilities differ by less than 1e-6 (the order of near-equal keys);
  * gate weights and probabilities within 1e-5 absolute;
  * per-token int8 codes and scales bit-exact;
  * align outputs bit-exact given the same ids (the oracle's ids are fed to
    the GPU align);
  * layer output relative L2 <= 2e-2 (bf16), 5e-2 (W8A8), 1e-4 (fp32), over
    the tokens whose routing agrees, and the same bar on each such token's
    own relative L2; every workload is checked over all of its tokens.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "i8": 5e-2, "f32": 1e-4, "i4": 2e-2, "i4a8": 5e-2}


def _moe():
    import routing_dispatch_expert_gate_amd as moe
    return moe


def to_dev(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


class Case:
    """Generated inputs of one workload, on host and device, plus oracle routing."""

    def __init__(self, spec, seed):
        self.spec = spec
        self.inp = moe_synth.make_inputs(spec, seed)
        i = self.inp
        self.x, self.wg, self.bias = to_dev(i.x), to_dev(i.wg), to_dev(i.bias)
        self.w13, self.w2, self.s13, self.s2 = to_dev(i.w13), to_dev(i.w2), to_dev(i.s13), to_dev(i.s2)
        if spec.w_dtype in ("i4", "i4a8") and self.w13 is not None:
            # int4 codes -> the kernels' packed layout (two per byte)
            self.w13, self.w2 = _moe().pack_int4(self.w13), _moe().pack_int4(self.w2)
        s = spec
        self.route = oracle.route(oracle.to_f64(i.x, s.x_dtype), oracle.to_f64(i.wg, s.wg_dtype), s.k, i.bias)
        self.C = oracle.capacity(s.T, s.k, s.E, s.capacity_factor)
        self.align = oracle.align(self.route["ids"], s.E, self.C)


_CACHE = {}


def config_case(cfg):
    if cfg not in _CACHE:
        print(f"[gpu-parity] generating workload {cfg}: {moe_synth.CONFIGS[cfg].name}", flush=True)
        _CACHE[cfg] = Case(moe_synth.CONFIGS[cfg], 1000 * cfg)
    return _CACHE[cfg]


def check_ids(ids_g, r):
    """Returns the boolean mask of rows whose ids agree exactly (after
    accepting order swaps of near-equal selected probabilities); asserts every
    other row lies in the near-tie band."""
    ids_o = r["ids"]
    same = (ids_g == ids_o).all(axis=1)
    bad = np.nonzero(~same)[0]
    band = r["gap_p"] < 1e-4
    swaps = 0
    for t in bad:
        if band[t]:
            continue
        # same set, order differs only between near-equal probabilities
        assert set(ids_g[t]) == set(ids_o[t]), (t, ids_g[t], ids_o[t], r["gap_p"][t])
        pg = r["p"][t, ids_g[t]]
        assert np.all(np.diff(pg) <= 1e-6), (t, ids_g[t], ids_o[t], pg)
        swaps += 1
    print(f"[ids] rows={len(ids_o)} mismatched={len(bad)} in-band={int(band[bad].sum())} "
          f"order-swaps={swaps} band-size={int(band.sum())}")
    return same


# ------------------------------------------------------------------ route
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_route_matches_oracle(cfg):
    moe = _moe()
    c = config_case(cfg)
    s = c.spec
    quant = s.w_dtype == "i8"
    r = moe.route(c.x, c.wg, s.k, bias=c.bias, want_p=True, quant=quant)
    torch.cuda.synchronize()
    print(moe.last_dispatch())
    ids_g = r["ids"].cpu().numpy()
    same = check_ids(ids_g, c.route)
    w_o = c.route["w"]
    p_o = c.route["p_sel"]
    assert np.abs(r["w"].cpu().numpy()[same] - w_o[same]).max() <= 1e-5
    assert np.abs(r["p"].cpu().numpy()[same] - p_o[same]).max() <= 1e-5
    np.testing.assert_allclose(r["w"].cpu().numpy().sum(axis=1), 1.0, atol=1e-5)
    if quant:
        xq_o, xs_o = oracle.quant_per_token_int8(moe_synth.bf16_bits_as_f32(c.inp.x))
        np.testing.assert_array_equal(r["xq"].cpu().numpy(), xq_o)
        np.testing.assert_array_equal(r["xs"].cpu().numpy(), xs_o)


@pytest.mark.parametrize("T,E,k,H", [(40, 8, 2, 256), (40, 16, 4, 128), (40, 64, 6, 2048), (40, 256, 8, 512),
                                     (8300, 64, 6, 512), (16400, 64, 6, 2048)])
def test_route_zero_rows_and_quant_edge_values(T, E, k, H):
    """A zero row routes to experts 0..k-1 with weight 1/k and gets scale 1;
    exact half quotients round half-even; the last two shapes take the
    fused E <= 64 kernel, with the edge rows in the first and last blocks."""
    moe = _moe()
    for base in ((0,) if T < 1000 else (0, T - 40)):
        spec = moe_synth.Spec("z", T, H, E, k, 64)
        i = moe_synth.make_inputs(spec, 7, with_experts=False)
        x = moe_synth.bf16_bits_as_f32(i.x)
        x[base + 3] = 0.0
        x[base + 5, :] = 0.0
        x[base + 5, 7] = -2.5                         # scale 2.5/127, code -127
        x[base + 6, :4] = [127.0, -63.5, 0.5, 1.5]    # exact .5 quotients round half-even
        xb = moe_synth.f32_to_bf16_bits(x)
        r = moe.route(to_dev(xb), to_dev(i.wg), k, want_p=True, quant=True)
        torch.cuda.synchronize()
        print(moe.last_dispatch())
        assert ("route_fused_kernel" in moe.last_dispatch()) == (T > 1000)
        ids = r["ids"].cpu().numpy()
        np.testing.assert_array_equal(ids[base + 3], np.arange(k))
        np.testing.assert_allclose(r["w"].cpu().numpy()[base + 3], 1.0 / k, atol=1e-7)
        xq_o, xs_o = oracle.quant_per_token_int8(moe_synth.bf16_bits_as_f32(xb))
        np.testing.assert_array_equal(r["xq"].cpu().numpy(), xq_o)
        np.testing.assert_array_equal(r["xs"].cpu().numpy(), xs_o)


# one case per router variant (the dispatch name is checked, so each case
# really takes its path): FMA for E <= 16 at ordinary and wide H, and the MFMA
# logits + top-k pair for E <= 64 (rank top-k; many tokens, ragged last tile,
# bias) and E > 64 (argmax rounds), with and without a K split
ROUTE_PATHS = [
    (moe_synth.Spec("fma_wide_bf16", 37, 8192, 8, 2, 64, wg_dtype="f32"), True, "route_fma_kernel"),
    (moe_synth.Spec("fma_wide_f32", 21, 6144, 4, 2, 64, x_dtype="f32", wg_dtype="f32"), True,
     "route_fma_kernel"),
    (moe_synth.Spec("fma_e16_f32x", 50, 4096, 16, 4, 64, x_dtype="f32"), True, "route_fma_kernel"),
    # one, four and sixteen tokens per workgroup (with a ragged last one)
    (moe_synth.Spec("fma_tb1_bias", 300, 2048, 8, 2, 64, zipf_s=1.1), True, "tokens/wg=1,"),
    (moe_synth.Spec("fma_tb4_e16", 2049, 1024, 12, 3, 64), True, "tokens/wg=4,"),
    (moe_synth.Spec("fma_tb16_e8", 4099, 512, 8, 2, 64, wg_dtype="f32"), False, "tokens/wg=16,"),
    (moe_synth.Spec("fma_tb16_many", 16411, 256, 8, 2, 64), True, "tokens/wg=16,"),
    # E <= 64, large batches: the fused kernel (logits on chip, x read once),
    # two parts of H (H <= 1024: 2, 4, 8 or 16 substeps per wave), four
    # (H = 2048) and eight (H = 4096), ragged last token block, bias, codes;
    # 8-wave workgroups (64 or 32 tokens) for two or four parts, 16 waves (32
    # tokens) for eight
    (moe_synth.Spec("e64_ragged_bias", 130 * 64 + 37, 256, 64, 6, 64, zipf_s=1.1), True,
     "route_fused_kernel(tokens/wg=64,parts=2)"),
    (moe_synth.Spec("e32_many_tokens", 128 * 64 + 1, 128, 32, 3, 64), False,
     "route_fused_kernel(tokens/wg=64,parts=2)"),
    (moe_synth.Spec("fused_e32_h512", 8200, 512, 32, 3, 64), False, "route_fused_kernel(tokens/wg=64,parts=2)"),
    (moe_synth.Spec("fused_e64_h2048_codes", 16384 + 77, 2048, 64, 6, 64, zipf_s=1.1), True,
     "route_fused_kernel(tokens/wg=32,parts=4)"),
    (moe_synth.Spec("fused_e48_h4096_codes", 2085, 4096, 48, 4, 64), True,
     "route_fused_kernel(tokens/wg=32,parts=8)"),
    (moe_synth.Spec("fused_e64_h4096", 2048, 4096, 64, 8, 64), False, "route_fused_kernel(tokens/wg=32,parts=8)"),
    # below 64 workgroups the batch keeps the K split
    (moe_synth.Spec("e64_h2048_splitk", 4000, 2048, 64, 6, 64), True, "route_gemm_kernel("),
    (moe_synth.Spec("logits_e64_splitk", 16, 4096, 64, 6, 64), True, "route_gemm_kernel("),
    (moe_synth.Spec("logits_e128", 300, 1024, 128, 4, 64), False, "route_gemm_kernel("),
    (moe_synth.Spec("logits_e256_T1", 1, 4096, 256, 8, 64), True, "route_gemm_kernel("),
    # one expert tile and no K split (ragged last tile), with codes
    (moe_synth.Spec("e48_codes_ragged", 1000, 128, 48, 6, 64, zipf_s=1.1), True, "route_gemm_kernel("),
    # large batches: 128 x 128 tiles split in K (ragged last token tile, codes
    # folded by two threads per row); E not a multiple of 128 keeps 64 x 64
    # (a full grid without a split; at E = 80 the second expert tile mostly
    # past E)
    (moe_synth.Spec("big_e256_codes", 4096 + 37, 512, 256, 8, 64), True,
     "tokens/wg=128,experts/wg=128,ksplit=4)"),
    (moe_synth.Spec("big_e64_codes", 16384 + 5, 1024, 64, 6, 64, zipf_s=1.1), True,
     "route_fused_kernel(tokens/wg=64,parts=2)"),
    (moe_synth.Spec("big_e80", 8300, 256, 80, 4, 64), False, "tokens/wg=64,experts/wg=64,ksplit=1)"),
]


@pytest.mark.parametrize("spec,quant,path", ROUTE_PATHS, ids=[p[0].name for p in ROUTE_PATHS])
def test_route_paths(spec, quant, path):
    moe = _moe()
    i = moe_synth.make_inputs(spec, 99, with_experts=False)
    r = moe.route(to_dev(i.x), to_dev(i.wg), spec.k, bias=to_dev(i.bias), want_p=True, quant=quant)
    torch.cuda.synchronize()
    print(moe.last_dispatch())
    d = moe.last_dispatch()
    assert path in d
    if spec.name in ("logits_e64_splitk", "logits_e128", "e64_h2048_splitk"):
        assert "ksplit=1)" not in d            # K really split
    ro = oracle.route(oracle.to_f64(i.x, spec.x_dtype), oracle.to_f64(i.wg, spec.wg_dtype), spec.k, i.bias)
    same = check_ids(r["ids"].cpu().numpy(), ro)
    assert np.abs(r["w"].cpu().numpy()[same] - ro["w"][same]).max() <= 1e-5
    assert np.abs(r["p"].cpu().numpy()[same] - ro["p_sel"][same]).max() <= 1e-5
    if quant:
        xf = i.x if spec.x_dtype == "f32" else moe_synth.bf16_bits_as_f32(i.x)
        xq_o, xs_o = oracle.quant_per_token_int8(xf)
        np.testing.assert_array_equal(r["xq"].cpu().numpy(), xq_o)
        np.testing.assert_array_equal(r["xs"].cpu().numpy(), xs_o)


# --------------------------------------------------- group-limited route
# (spec, n_group, topk_group, quant): DeepSeek-V3-like 256 experts in 8
# groups with 4 kept; 160 experts in 8 groups of 20 with 3 kept (groups that
# straddle lanes); one kept group of 8 (k = 6 inside it); groups of one
GROUPED = [
    (moe_synth.Spec("g_e160_G8_TG3", 300, 512, 160, 6, 64, zipf_s=1.1), 8, 3, True),
    (moe_synth.Spec("g_e64_G8_TG1", 257, 1024, 64, 6, 64), 8, 1, False),
    (moe_synth.Spec("g_e32_G32_TG5_T1", 1, 256, 32, 4, 64), 32, 5, True),
    (moe_synth.Spec("g_e256_G8_TG4_splitk", 64, 4096, 256, 8, 64), 8, 4, False),
    # a batch the plain router takes fused: the grouped one keeps two kernels
    (moe_synth.Spec("g_e64_G8_TG3_bigT", 8300, 256, 64, 6, 64, zipf_s=1.1), 8, 3, True),
]


def _check_grouped(r, ro):
    """ids parity with near ties exempt: the k-th/next candidate gap or the
    kept/next group-score gap below 1e-4 (fp32 logits vs the fp64 oracle)."""
    band = dict(ro, gap_p=np.minimum(ro["gap_p"], ro["gap_group"]))
    ids_g = r["ids"].cpu().numpy()
    same = check_ids(ids_g, band)
    assert np.abs(r["w"].cpu().numpy()[same] - ro["w"][same]).max() <= 1e-5
    if r["p"] is not None:
        assert np.abs(r["p"].cpu().numpy()[same] - ro["p_sel"][same]).max() <= 1e-5
    # every row, exempt or not: ids distinct, inside at most topk_group groups
    return same


@pytest.mark.parametrize("spec,G,TG,quant", GROUPED, ids=[g[0].name for g in GROUPED])
def test_route_grouped_matches_oracle(spec, G, TG, quant):
    moe = _moe()
    i = moe_synth.make_inputs(spec, 77, with_experts=False)
    r = moe.route(to_dev(i.x), to_dev(i.wg), spec.k, bias=to_dev(i.bias), want_p=True, quant=quant,
                  n_group=G, topk_group=TG)
    torch.cuda.synchronize()
    d = moe.last_dispatch()
    print(d)
    assert "<grouped>" in d
    ro = oracle.route_grouped(oracle.to_f64(i.x, spec.x_dtype), oracle.to_f64(i.wg, spec.wg_dtype), spec.k, G,
                              TG, i.bias)
    _check_grouped(r, ro)
    ids = r["ids"].cpu().numpy()
    gsz = spec.E // G
    for t in range(spec.T):
        assert len(set(ids[t].tolist())) == spec.k
        assert len(set((ids[t] // gsz).tolist())) <= TG
    if quant:
        xq_o, xs_o = oracle.quant_per_token_int8(moe_synth.bf16_bits_as_f32(i.x))
        np.testing.assert_array_equal(r["xq"].cpu().numpy(), xq_o)
        np.testing.assert_array_equal(r["xs"].cpu().numpy(), xs_o)


def test_route_grouped_on_fine_grained_workload():
    """The 4096-token, 256-expert, top-8 workload with 8 groups and 4 kept."""
    moe = _moe()
    c = config_case(3)
    s = c.spec
    r = moe.route(c.x, c.wg, s.k, bias=c.bias, want_p=True, n_group=8, topk_group=4)
    torch.cuda.synchronize()
    ro = oracle.route_grouped(oracle.to_f64(c.inp.x, s.x_dtype), oracle.to_f64(c.inp.wg, s.wg_dtype), s.k, 8, 4,
                              c.inp.bias)
    same = _check_grouped(r, ro)
    # the group limit really changes the routing of some tokens
    assert (ro["ids"] != c.route["ids"]).any(axis=1).sum() > 0
    assert same.mean() > 0.99


def test_route_grouped_all_groups_equals_plain_route():
    """topk_group == n_group: bit-identical to moe_route (same arithmetic)."""
    moe = _moe()
    spec = moe_synth.Spec("g_all", 300, 1024, 256, 8, 64)
    i = moe_synth.make_inputs(spec, 5, with_experts=False)
    a = moe.route(to_dev(i.x), to_dev(i.wg), 8, bias=to_dev(i.bias), want_p=True)
    b = moe.route(to_dev(i.x), to_dev(i.wg), 8, bias=to_dev(i.bias), want_p=True, n_group=8, topk_group=8)
    torch.cuda.synchronize()
    assert torch.equal(a["ids"], b["ids"])
    assert torch.equal(a["w"], b["w"]) and torch.equal(a["p"], b["p"])


# ---------------------------------------------------------- route + align
ROUTE_ALIGN = [
    # spec, capacity, block_m, quant, fused
    (moe_synth.Spec("ra_e256_T16", 16, 4096, 256, 8, 64), 0, 64, True, True),
    (moe_synth.Spec("ra_e64_T64_cap", 64, 1024, 64, 6, 64, zipf_s=1.1), 7, 64, False, True),
    (moe_synth.Spec("ra_e32_T1", 1, 256, 32, 4, 64), 0, 16, True, True),
    (moe_synth.Spec("ra_e8_T16_f32wg", 16, 4096, 8, 2, 64, wg_dtype="f32"), 0, 64, False, True),
    (moe_synth.Spec("ra_e16_T10_cap", 10, 256, 16, 4, 64, x_dtype="f32", wg_dtype="f32"), 2, 32, True, True),
    (moe_synth.Spec("ra_e64_T300", 300, 512, 64, 6, 64), 30, 128, False, False),
    (moe_synth.Spec("ra_e8_T100", 100, 512, 8, 2, 64), 0, 256, True, False),
    # large batches at E <= 64: the route kernel publishes per-workgroup
    # counts and one align launch takes them (fused E <= 64 router, FMA router)
    (moe_synth.Spec("ra_e64_T8300_cap", 8300, 256, 64, 6, 64, zipf_s=1.1), 700, 128, True, False),
    (moe_synth.Spec("ra_e16_T20011_cap", 20011, 128, 16, 4, 64, zipf_s=1.1), 4000, 256, False, False),
    # E > 64 (MFMA logits + top-k): the top-k workgroups publish the counts;
    # T not a multiple of their 16 tokens, E = 80 (three count sums per
    # expert per align thread), codes with the small-batch top-k
    (moe_synth.Spec("ra_e256_T4100_cap", 4100, 256, 256, 8, 64, zipf_s=1.1), 150, 128, False, False),
    (moe_synth.Spec("ra_e128_T700_q", 700, 512, 128, 6, 64), 0, 64, True, False),
    (moe_synth.Spec("ra_e80_T1000_cap", 1000, 256, 80, 6, 64, zipf_s=1.1), 60, 32, False, False),
]


@pytest.mark.parametrize("spec,C,bm,quant,fused", ROUTE_ALIGN, ids=[r[0].name for r in ROUTE_ALIGN])
def test_route_align_equals_route_then_align(spec, C, bm, quant, fused):
    """moe_route_align gives exactly the outputs of moe_route followed by
    moe_align (one launch where one workgroup takes every token), and those
    match the oracle."""
    moe = _moe()
    i = moe_synth.make_inputs(spec, 31, with_experts=False)
    x, wg, b = to_dev(i.x), to_dev(i.wg), to_dev(i.bias)
    ra = moe.route_align(x, wg, spec.k, capacity=C, block_m=bm, bias=b, want_p=True, quant=quant)
    torch.cuda.synchronize()
    d = moe.last_dispatch()
    print(d)
    assert ("(one launch)" in d) == fused, d
    # batches of at least 4096 slots take the align step from the route
    # step's published counts
    assert ("from route counts" in d) == (not fused and spec.T * spec.k >= 4096), d
    r = moe.route(x, wg, spec.k, bias=b, want_p=True, quant=quant)
    a = moe.align(r["ids"], spec.E, C, bm)
    torch.cuda.synchronize()
    for key in ("ids", "w", "p") + (("xq", "xs") if quant else ()):
        assert torch.equal(ra[key], r[key]), key
    nt = int(a["num_tiles"].item())
    assert int(ra["num_tiles"].item()) == nt
    for key in ("counts", "offsets", "sorted_slot", "pos", "num_dropped"):
        assert torch.equal(ra[key], a[key]), key
    assert torch.equal(ra["tiles"][:nt], a["tiles"][:nt]) and (ra["tiles"][nt:, 0] == -1).all()
    ro = oracle.route(oracle.to_f64(i.x, spec.x_dtype), oracle.to_f64(i.wg, spec.wg_dtype), spec.k, i.bias)
    check_ids(ra["ids"].cpu().numpy(), ro)
    al = oracle.align(ra["ids"].cpu().numpy(), spec.E, C or None)
    np.testing.assert_array_equal(ra["pos"].cpu().numpy(), al["pos"])
    np.testing.assert_array_equal(ra["sorted_slot"].cpu().numpy(), al["sorted_slot"])
    np.testing.assert_array_equal(ra["offsets"].cpu().numpy(), al["offsets"])


# ------------------------------------------------------------------ align
def _check_align(ids, E, C, bm):
    moe = _moe()
    a = moe.align(to_dev(ids.astype(np.int32)), E, C or 0, bm)
    torch.cuda.synchronize()
    # up to 2^14 slots one workgroup does all three steps, above them three launches
    assert ("align_one_block_kernel" in moe.last_dispatch()) == (ids.size <= 1 << 14), moe.last_dispatch()
    ref = oracle.align(ids, E, C)
    np.testing.assert_array_equal(a["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(a["offsets"].cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(a["sorted_slot"].cpu().numpy(), ref["sorted_slot"])
    np.testing.assert_array_equal(a["pos"].cpu().numpy(), ref["pos"])
    assert int(a["num_dropped"].item()) == ref["num_dropped"]
    nt = int(a["num_tiles"].item())
    tl = a["tiles"].cpu().numpy()
    assert [tuple(v) for v in tl[:nt, :3]] == oracle.tiles(ref["offsets"], bm)
    assert (tl[nt:, 0] == -1).all() and (tl[:nt, 3] == 0).all()
    return a


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_align_bit_exact_on_workloads(cfg):
    moe = _moe()
    c = config_case(cfg)
    s = c.spec
    bm = moe.ffn_block_m(s.T, s.H, s.I, s.E, s.k, {"f32": torch.float32, "bf16": torch.bfloat16,
                                                    "i8": torch.int8}[s.w_dtype])
    _check_align(c.route["ids"], s.E, c.C, bm)
    print(f"N={c.align['offsets'][-1]} dropped={c.align['num_dropped']}")


@pytest.mark.parametrize("T,E,k,C,bm,skew", [
    (1, 8, 2, None, 128, 0.0), (3000, 8, 3, None, 128, 0.0), (1000, 64, 6, 30, 64, 1.5),
    (5000, 256, 8, 120, 128, 0.0), (4097, 256, 8, None, 256, 0.0), (2048, 4, 1, 100, 16, 3.0),
    (999, 1, 1, 500, 32, 0.0), (700, 7, 7, 650, 128, 0.0), (20000, 64, 6, 1920, 128, 1.1),
    (2048, 256, 8, 80, 128, 0.0), (2049, 8, 8, None, 256, 0.0), (40000, 64, 6, 4000, 64, 1.1),
    (4096, 4, 4, None, 16, 2.0),
])
def test_align_bit_exact_edge_cases(T, E, k, C, bm, skew):
    rng = np.random.default_rng(T * 31 + E)
    pri = 1.0 / np.arange(1, E + 1) ** skew
    pri = pri / pri.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=pri) for _ in range(T)])
    _check_align(ids, E, C, bm)


def test_align_all_tokens_to_one_expert_keeps_first_c():
    T, E, k, C = 3000, 16, 2, 700
    ids = np.tile(np.array([[5, 9]]), (T, 1))
    a = _check_align(ids, E, C, 128)
    pos = a["pos"].cpu().numpy()
    np.testing.assert_array_equal(pos[:, 0] >= 0, np.arange(T) < C)


def test_align_is_deterministic():
    moe = _moe()
    for cfg in (3, 5):
        c = config_case(cfg)
        s = c.spec
        ids = to_dev(c.route["ids"])
        first = None
        for _ in range(100):
            a = moe.align(ids, s.E, c.C or 0, 128)
            snap = [a[n].cpu().numpy().copy() for n in ("counts", "offsets", "sorted_slot", "pos", "tiles")]
            if first is None:
                first = snap
            else:
                for u, v in zip(first, snap):
                    np.testing.assert_array_equal(u, v)


# --------------------------------------------------------- FFN + combine
def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _check_out(name, got, ref, keep, tol):
    """Aggregate relative L2 over the kept tokens, and each kept token's own
    relative L2 (tokens whose reference row is all zero, i.e. every slot
    dropped, must be exactly zero)."""
    rel = _rel(got[keep], ref[keep])
    nrm = np.linalg.norm(ref, axis=1)
    err = np.linalg.norm(got - ref, axis=1)
    live = keep & (nrm > 0)
    per = err[live] / nrm[live]
    worst = float(per.max()) if per.size else 0.0
    print(f"[{name}] rel-L2 {rel:.3e} over {int(keep.sum())}/{len(keep)} tokens; worst token {worst:.3e}")
    assert rel <= tol, rel
    assert worst <= tol, (worst, int(np.nonzero(live)[0][np.argmax(per)]))
    dead = keep & (nrm == 0)
    assert np.all(got[dead] == 0)


def _ffn_combine_case(c, sample):
    """GPU align -> expert FFN -> combine on the oracle's routing; compare with
    the oracle layer on ``sample``."""
    moe = _moe()
    s = c.spec
    wdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8, "i4": torch.uint8,
           "i4a8": "w4a8"}[s.w_dtype]
    a8 = s.w_dtype in ("i8", "i4a8")
    bm = moe.ffn_block_m(s.T, s.H, s.I, s.E, s.k, wdt)
    ids = to_dev(c.route["ids"])
    w = to_dev(c.route["w"].astype(np.float32))
    a = moe.align(ids, s.E, c.C or 0, bm)
    if a8:
        xq, xs = oracle.quant_per_token_int8(moe_synth.bf16_bits_as_f32(c.inp.x))
        act, xs_d = to_dev(xq), to_dev(xs)
    else:
        act, xs_d = c.x, None
    w4a8 = s.w_dtype == "i4a8"
    y = moe.expert_ffn(act, c.w13, c.w2, a["sorted_slot"], a["tiles"], a["num_tiles"], bm, s.k,
                       topk_w=w, xs=xs_d, s13=c.s13, s2=c.s2, w4a8=w4a8)
    out = moe.combine(y, a["pos"], None, s.T, s.k, torch.float32 if s.out_dtype == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    print(moe.last_dispatch())
    ref = oracle.layer_from_inputs(c.inp, sample_tokens=sample)
    got = out.float().cpu().numpy().astype(np.float64)[sample]
    every = np.ones(len(sample), dtype=bool)
    _check_out(f"ffn+combine {s.name}", got, ref["out"], every, TOL[s.w_dtype])
    # weighted combine path (rows unweighted, weights applied in combine)
    y2 = moe.expert_ffn(act, c.w13, c.w2, a["sorted_slot"], a["tiles"], a["num_tiles"], bm, s.k,
                        topk_w=None, xs=xs_d, s13=c.s13, s2=c.s2, w4a8=w4a8)
    out2 = moe.combine(y2, a["pos"], w, s.T, s.k, torch.float32 if s.out_dtype == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    got2 = out2.float().cpu().numpy().astype(np.float64)[sample]
    _check_out(f"ffn+combine weighted {s.name}", got2, ref["out"], every, TOL[s.w_dtype])


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_ffn_combine_on_workloads(cfg):
    c = config_case(cfg)
    _ffn_combine_case(c, np.arange(c.spec.T))


SMALL = [
    moe_synth.Spec("bf16_E16_I192_cap1", 300, 256, 16, 4, 192, capacity_factor=1.0),
    moe_synth.Spec("bf16_E64_T777_cap1.25", 777, 512, 64, 6, 256, capacity_factor=1.25),
    moe_synth.Spec("bf16_E32_H320", 129, 320, 32, 3, 128),
    moe_synth.Spec("bf16_E256_T200_k8", 200, 256, 256, 8, 128, capacity_factor=1.25),
    moe_synth.Spec("i8_E16_zipf_cap", 500, 256, 16, 2, 384, w_dtype="i8", capacity_factor=1.25, zipf_s=1.1),
    moe_synth.Spec("i8_E64_T300", 300, 384, 64, 6, 256, w_dtype="i8"),
    moe_synth.Spec("f32_E4_H192", 100, 192, 4, 2, 128, x_dtype="f32", wg_dtype="f32", w_dtype="f32",
                   out_dtype="f32"),
    moe_synth.Spec("bf16_E1_k1", 200, 128, 1, 1, 128),
    moe_synth.Spec("bf16_k_eq_E", 90, 128, 4, 4, 64, wg_dtype="f32"),
    moe_synth.Spec("bf16_T1_E256", 1, 512, 256, 8, 128),
    # the smallest hidden sizes the limits allow (H = I = 64), and H = 64 with fp32
    moe_synth.Spec("bf16_H64_I64", 100, 64, 4, 2, 64, capacity_factor=1.25),
    moe_synth.Spec("f32_H64_I128", 70, 64, 8, 3, 128, x_dtype="f32", wg_dtype="f32", w_dtype="f32",
                   out_dtype="f32"),
    moe_synth.Spec("i4_H128_I64", 90, 128, 4, 2, 64, w_dtype="i4"),
    # prefill tiles with a mostly empty last round: the down GEMM splits that
    # round's units over K (partial tiles summed by the reduce kernel)
    moe_synth.Spec("bf16_prefill_last_round_split", 1024, 512, 4, 2, 512),
    moe_synth.Spec("i8_prefill_last_round_split", 1024, 512, 4, 2, 512, w_dtype="i8"),
    # W4A16: one case per int4 tile (prefill/mid 256 x BN, decode 64 x BN, for
    # BN = 256, 128 and 64), with and without drops
    moe_synth.Spec("i4_prefill_E4", 600, 512, 4, 2, 384, w_dtype="i4"),
    moe_synth.Spec("i4_mid_H320_I192_cap1", 257, 320, 8, 2, 192, w_dtype="i4", capacity_factor=1.0),
    moe_synth.Spec("i4_decode_E64", 16, 512, 64, 6, 256, w_dtype="i4"),
    moe_synth.Spec("i4_decode_H384_I192", 8, 384, 32, 4, 192, w_dtype="i4"),
    moe_synth.Spec("i4_decode_H320", 8, 320, 16, 2, 128, w_dtype="i4", zipf_s=1.1),
    moe_synth.Spec("i4_mid_E8_T512", 512, 512, 8, 2, 256, w_dtype="i4"),
    moe_synth.Spec("i4_prefill_H384_I192", 1024, 384, 4, 2, 192, w_dtype="i4"),
    moe_synth.Spec("i4_prefill_H320_k1", 800, 320, 4, 1, 128, w_dtype="i4", capacity_factor=1.25),
    # W4A8: the int8 MFMA path on packed int4 weights (prefill, mid, decode;
    # BN = 256 and 128; H and I multiples of 128)
    moe_synth.Spec("i4a8_prefill_E4", 600, 512, 4, 2, 384, w_dtype="i4a8"),
    moe_synth.Spec("i4a8_mid_H384_cap1", 300, 384, 8, 2, 256, w_dtype="i4a8", capacity_factor=1.0, zipf_s=1.1),
    moe_synth.Spec("i4a8_decode_E64", 16, 512, 64, 6, 256, w_dtype="i4a8"),
    moe_synth.Spec("i4a8_decode_H384", 8, 384, 32, 4, 128, w_dtype="i4a8"),
    # large batches whose route step publishes per-workgroup counts
    # and whose align step is one launch over them, with capacity drops
    moe_synth.Spec("align_from_route_e64_cap", 8300, 256, 64, 6, 128, capacity_factor=1.0, zipf_s=1.1),
    moe_synth.Spec("align_from_route_e32_i8_cap", 9001, 128, 32, 3, 128, w_dtype="i8", capacity_factor=1.25,
                   zipf_s=1.1),
    moe_synth.Spec("align_from_route_e16_fma_cap", 20011, 128, 16, 4, 64, capacity_factor=1.25, zipf_s=1.1),
    # E > 64: counts from the top-k workgroups of the MFMA router
    moe_synth.Spec("align_from_route_e256_cap", 4100, 256, 256, 8, 128, capacity_factor=1.25, zipf_s=1.1),
    moe_synth.Spec("align_from_route_e128_i8", 700, 256, 128, 6, 128, w_dtype="i8"),
]


@pytest.mark.parametrize("spec", SMALL, ids=[s.name for s in SMALL])
def test_ffn_combine_small_shapes(spec):
    _ffn_combine_case(Case(spec, 4242), np.arange(spec.T))


# -------------------------------------------------------- combine + shared
COMBINE_SHARED = [
    # T, H, E, k, C, y dtype, out dtype, shared, bias, in place
    (257, 192, 8, 2, 60, "bf16", "bf16", True, True, False),
    (130, 256, 16, 3, 0, "f32", "f32", True, False, False),
    (64, 128, 64, 8, 9, "bf16", "f32", False, True, False),
    (300, 320, 4, 1, 70, "f32", "bf16", True, True, True),
    (33, 64, 32, 6, 2, "bf16", "bf16", True, True, True),   # almost every slot dropped
]


@pytest.mark.parametrize("case", COMBINE_SHARED, ids=lambda c: "T%d_H%d_k%d_%s_%s" % (c[0], c[1], c[3], c[5], c[6]))
def test_combine_shared_matches_oracle(case):
    """moe_combine_shared against the oracle's combine_shared, element by
    element: routed sum in slot order + factor * S + b, fp32 on the GPU."""
    moe = _moe()
    T, H, E, k, C, ydt, odt, with_s, with_b, in_place = case
    rng = np.random.default_rng(T * 1000 + H)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    al = oracle.align(ids, E, C)
    pos = al["pos"].reshape(T, k)
    N = max(int(al["offsets"][-1]), 1)
    y = rng.standard_normal((N, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    S = rng.standard_normal((T, H)).astype(np.float32) if with_s else None
    b = rng.standard_normal(H).astype(np.float32) if with_b else None
    f = -0.625
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    y_d = torch.from_numpy(y).cuda().to(tdt[ydt])
    S_d = torch.from_numpy(S).cuda().to(tdt[odt]) if with_s else None
    # the oracle sees exactly the stored values
    y64 = y_d.float().cpu().numpy().astype(np.float64)
    S64 = S_d.float().cpu().numpy().astype(np.float64) if with_s else None
    ref = oracle.combine_shared(y64, pos, w.astype(np.float64), S64, f, b)
    out = S_d if in_place else None
    got = moe.combine_shared(y_d, to_dev(al["pos"].astype(np.int32)), to_dev(w), T, k, tdt[odt], shared=S_d,
                             shared_factor=f, bias=to_dev(b), out=out)
    if in_place:
        assert got.data_ptr() == S_d.data_ptr()
    torch.cuda.synchronize()
    print(moe.last_dispatch())
    g = got.float().cpu().numpy().astype(np.float64)
    # fp32 accumulation of k+2 terms, then one rounding to the output dtype
    mag = np.zeros((T, H))
    for j in range(k):
        keep = pos[:, j] >= 0
        mag[keep] += np.abs(w[keep, j, None] * y64[pos[keep, j]])
    if with_s:
        mag += abs(f) * np.abs(S64)
    if with_b:
        mag += np.abs(b)[None, :]
    out_eps = 2.0 ** -8 if odt == "bf16" else 2.0 ** -24
    bound = out_eps * np.abs(ref) + (k + 2) * 2.0 ** -24 * mag * (1 + out_eps) + 1e-30
    err = np.abs(g - ref)
    assert np.all(err <= bound), (float((err / bound).max()), np.unravel_index(np.argmax(err / bound), err.shape))
    # tokens with every slot dropped get exactly the rounded factor * S + b
    dead = np.all(pos < 0, axis=1)
    if dead.any() and not with_s and not with_b:
        assert np.all(g[dead] == 0)


def test_combine_shared_without_extras_equals_combine():
    moe = _moe()
    rng = np.random.default_rng(5)
    T, H, E, k = 200, 256, 16, 4
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    al = oracle.align(ids, E, 40)
    y = torch.from_numpy(rng.standard_normal((int(al["offsets"][-1]), H)).astype(np.float32)).cuda().bfloat16()
    w = to_dev(rng.random((T, k)).astype(np.float32))
    p = to_dev(al["pos"].astype(np.int32))
    a = moe.combine(y, p, w, T, k, torch.bfloat16)
    b = moe.combine_shared(y, p, w, T, k, torch.bfloat16, shared=None, shared_factor=3.0, bias=None)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# --------------------------------------------------------------- W4A16
def test_pack_int4_layout():
    """Packed byte j of a row = code 2j (low nibble) | code 2j+1 (high
    nibble), two's complement nibbles; checked against that definition."""
    moe = _moe()
    rng = np.random.default_rng(8)
    codes = rng.integers(-8, 8, size=(37, 192), dtype=np.int8)
    got = moe.pack_int4(to_dev(codes)).cpu().numpy()
    lo = codes[:, 0::2].astype(np.int64) & 0xF
    hi = codes[:, 1::2].astype(np.int64) & 0xF
    np.testing.assert_array_equal(got, (lo | (hi << 4)).astype(np.uint8))


def test_w4a8_skewed_workload():
    """The skewed 16384-token, 64-expert workload with int4 weights and int8
    activations (W4A8), on a token sample."""
    spec = moe_synth.CONFIGS[5].replace(name="skewed_w4a8_T16384_H2048_E64_k6_I1408_cap1.25", w_dtype="i4a8")
    _layer_case(Case(spec, 5000), np.arange(spec.T))


def test_w4a16_decode_workload():
    """The 16-token, 256-expert, top-8 decode workload with int4 experts."""
    spec = moe_synth.CONFIGS[4].replace(name="decode_w4a16_T16_H4096_E256_k8_I1024", w_dtype="i4")
    _layer_case(Case(spec, 4000), np.arange(spec.T))


# ------------------------------------------------------------------ layer
def _layer_case(c, sample, check_aux=True):
    moe = _moe()
    s = c.spec
    T, k = s.T, s.k
    aux = {
        "topk_ids": torch.empty((T, k), dtype=torch.int32, device="cuda"),
        "topk_w": torch.empty((T, k), dtype=torch.float32, device="cuda"),
        "topk_p": torch.empty((T, k), dtype=torch.float32, device="cuda"),
        "counts": torch.empty(s.E, dtype=torch.int32, device="cuda"),
        "offsets": torch.empty(s.E + 1, dtype=torch.int32, device="cuda"),
        "pos": torch.empty((T, k), dtype=torch.int32, device="cuda"),
        "sorted_slot": torch.empty(T * k, dtype=torch.int32, device="cuda"),
        "num_dropped": torch.empty(1, dtype=torch.int32, device="cuda"),
    }
    out = moe.layer(c.x, c.wg, c.w13, c.w2, k, capacity=c.C or 0, bias=c.bias, s13=c.s13, s2=c.s2, aux=aux,
                    w4a8=s.w_dtype == "i4a8")
    torch.cuda.synchronize()
    print(moe.last_dispatch())
    ids_g = aux["topk_ids"].cpu().numpy()
    same = check_ids(ids_g, c.route)
    pos_g = aux["pos"].cpu().numpy()
    agree = same & ((pos_g >= 0) == (c.align["pos"] >= 0)).all(axis=1)
    if same.all() and check_aux:
        np.testing.assert_array_equal(aux["counts"].cpu().numpy(), c.align["counts"])
        np.testing.assert_array_equal(aux["offsets"].cpu().numpy(), c.align["offsets"])
        np.testing.assert_array_equal(pos_g, c.align["pos"])
        np.testing.assert_array_equal(aux["sorted_slot"].cpu().numpy(), c.align["sorted_slot"])
        assert int(aux["num_dropped"].item()) == c.align["num_dropped"]
    assert agree.mean() > 0.99
    ref = oracle.layer_from_inputs(c.inp, sample_tokens=sample)
    keep = agree[sample]
    got = out.float().cpu().numpy().astype(np.float64)[sample]
    _check_out(f"layer {s.name}", got, ref["out"], keep, TOL[s.w_dtype])
    # every slot dropped -> exactly zero (the residual is the caller's)
    full_drop = (pos_g < 0).all(axis=1)
    if full_drop.any():
        assert float(out[torch.from_numpy(np.nonzero(full_drop)[0]).cuda()].abs().max()) == 0.0
    return out


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_layer_matches_oracle(cfg):
    c = config_case(cfg)
    _layer_case(c, np.arange(c.spec.T))


@pytest.mark.parametrize("spec", SMALL, ids=[s.name for s in SMALL])
def test_layer_small_shapes(spec):
    _layer_case(Case(spec, 4343), np.arange(spec.T))


def test_layer_is_deterministic_and_permutation_equivariant():
    moe = _moe()
    spec = moe_synth.Spec("perm", 512, 256, 16, 2, 128)
    c = Case(spec, 99)
    a = moe.layer(c.x, c.wg, c.w13, c.w2, spec.k)
    b = moe.layer(c.x, c.wg, c.w13, c.w2, spec.k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(spec.T)).cuda()
    p = moe.layer(c.x[perm].contiguous(), c.wg, c.w13, c.w2, spec.k)
    torch.cuda.synchronize()
    assert _rel(p.float().cpu().numpy(), a[perm].float().cpu().numpy()) < 1e-2


GRAPH_CASES = [
    moe_synth.Spec("graph_bf16_E64_cap", 300, 512, 64, 6, 256, capacity_factor=1.0),
    moe_synth.Spec("graph_w8a8_E16", 257, 256, 16, 2, 256, w_dtype="i8", capacity_factor=1.25),
    moe_synth.Spec("graph_w4a8_decode", 16, 512, 64, 6, 256, w_dtype="i4a8"),
]


@pytest.mark.parametrize("spec", GRAPH_CASES, ids=[s.name for s in GRAPH_CASES])
def test_layer_replays_from_a_hip_graph(spec):
    """moe_layer allocates nothing and enqueues only kernels, so a captured
    graph of it replays the eager result bit for bit, replay after replay,
    with other eager work (another layer call on other inputs) in between."""
    moe = _moe()
    c = Case(spec, 2024)
    other = Case(spec.replace(name=spec.name + "_other"), 2025)
    w4a8 = spec.w_dtype == "i4a8"
    L = moe.Layer(spec.T, spec.H, spec.I, spec.E, spec.k, c.x.dtype, "w4a8" if w4a8 else c.w13.dtype)
    out = torch.empty((spec.T, spec.H), dtype=c.x.dtype, device="cuda")
    C = c.C or 0

    def call(case, dst):
        L(case.x, case.wg, case.w13, case.w2, C, case.bias, case.s13, case.s2, out=dst)

    ref = torch.empty_like(out)
    call(c, ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(c, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(c, out)
    scratch = torch.empty_like(out)
    for i in range(3):
        out.zero_()
        call(other, scratch)            # eager work on the same workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref), f"replay {i}"
    ref_other = moe.layer(other.x, other.wg, other.w13, other.w2, spec.k, capacity=C, bias=other.bias,
                          s13=other.s13, s2=other.s2, w4a8=w4a8)
    torch.cuda.synchronize()
    assert torch.equal(scratch, ref_other)


@pytest.mark.parametrize("spec", [GRAPH_CASES[0], GRAPH_CASES[1],
                                  moe_synth.Spec("events_from_route_E8", 2048, 256, 8, 2, 256)],
                         ids=["bf16_E64_cap", "w8a8_E16", "from_route_E8"])
def test_layer_stage_events_time_each_step(spec):
    """moe_layer_aux.stage_events: the layer records the caller's six events
    around its five steps; the output is the same as without them, and the
    five intervals are non-negative and add up to the whole call."""
    moe = _moe()
    c = Case(spec, 77)
    L = moe.Layer(spec.T, spec.H, spec.I, spec.E, spec.k, c.x.dtype, c.w13.dtype)
    C = c.C or 0
    ref = L(c.x, c.wg, c.w13, c.w2, C, c.bias, c.s13, c.s2)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    ev_some = [evs[0].cuda_event, None, evs[2].cuda_event, None, None, evs[5].cuda_event]
    out_some = L(c.x, c.wg, c.w13, c.w2, C, c.bias, c.s13, c.s2, aux={"stage_events": ev_some})
    torch.cuda.synchronize()
    assert torch.equal(out_some.view(torch.int16), ref.view(torch.int16))
    out = L(c.x, c.wg, c.w13, c.w2, C, c.bias, c.s13, c.s2, aux={"stage_events": [e.cuda_event for e in evs]})
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    steps = [evs[j].elapsed_time(evs[j + 1]) for j in range(5)]
    total = evs[0].elapsed_time(evs[5])
    assert all(t >= 0 for t in steps), steps
    assert abs(sum(steps) - total) <= 1e-3 + 1e-3 * total, (steps, total)


def test_empty_batch_is_a_noop():
    moe = _moe()
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    wg = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    w13 = torch.zeros((8, 128, 128), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((8, 128, 64), dtype=torch.bfloat16, device="cuda")
    out = moe.layer(x, wg, w13, w2, 2)
    torch.cuda.synchronize()
    assert out.shape == (0, 128)
    assert moe.last_dispatch() == "none (T=0)"


# ------------------------------------------- layer with gate/sum options
# (spec, n_group, topk_group, shared, shared_factor, out_bias, in place):
# group-limited routing with a shared expert and an output bias in one call
LAYER_EX = [
    (moe_synth.Spec("lx_e64_G8_TG3_cap", 200, 256, 64, 6, 128, capacity_factor=1.25, zipf_s=1.0),
     8, 3, True, 0.5, True, False),
    (moe_synth.Spec("lx_e32_G4_TG2_i8_cap", 130, 256, 32, 4, 128, w_dtype="i8", capacity_factor=1.25),
     4, 2, True, 1.0, False, True),
    (moe_synth.Spec("lx_e64_plain_w4a8", 96, 256, 64, 4, 128, w_dtype="i4a8"), 0, 0, True, 2.0, True, False),
    (moe_synth.Spec("lx_e256_G8_TG4_T1", 1, 512, 256, 8, 128), 8, 4, False, 1.0, True, False),
    (moe_synth.Spec("lx_e256_G8_TG4_w4a16", 64, 512, 256, 8, 128, w_dtype="i4"), 8, 4, True, -1.0, True, True),
    # large batch at E = 64: the grouped router keeps two kernels (and its
    # workspace) where the plain one would be fused
    (moe_synth.Spec("lx_e64_G8_TG3_bigT_i8", 8300, 256, 64, 6, 128, w_dtype="i8", capacity_factor=1.25),
     8, 3, True, 0.5, True, False),
]


@pytest.mark.parametrize("case", LAYER_EX, ids=[c[0].name for c in LAYER_EX])
def test_layer_ex_matches_composition_and_oracle(case):
    """moe_layer_ex is bit for bit its steps called one by one (grouped route,
    align, expert FFN, combine with the shared term and bias), and matches
    the oracle layer with the same options on every token whose routing the
    fp32 logits decide as the fp64 oracle does."""
    moe = _moe()
    spec, G, TG, with_s, f, with_b, in_place = case
    c = Case(spec, 5151)
    s = c.spec
    T, H, k = s.T, s.H, s.k
    rng = np.random.default_rng(T + 17 * s.E)
    S = moe_synth.f32_to_bf16_bits((0.01 * rng.standard_normal((T, H))).astype(np.float32)) if with_s else None
    b = (0.01 * rng.standard_normal(H)).astype(np.float32) if with_b else None
    S_d, b_d = to_dev(S), to_dev(b)
    opts = dict(n_group=G, topk_group=TG, shared=S_d, shared_factor=f, out_bias=b_d)
    aux = {"topk_ids": torch.empty((T, k), dtype=torch.int32, device="cuda"),
           "pos": torch.empty((T, k), dtype=torch.int32, device="cuda")}
    w4a8 = s.w_dtype == "i4a8"
    a8 = s.w_dtype in ("i8", "i4a8")
    out_buf = S_d.clone() if in_place else None
    if in_place:
        opts["shared"] = out_buf
    L = moe.Layer(T, H, s.I, s.E, k, c.x.dtype, "w4a8" if w4a8 else c.w13.dtype)
    out = L(c.x, c.wg, c.w13, c.w2, capacity=c.C or 0, bias=c.bias, s13=c.s13, s2=c.s2, out=out_buf, aux=aux,
            options=opts)
    torch.cuda.synchronize()
    d = moe.last_dispatch()
    print(d)
    assert ("<grouped>" in d) == (G > 0)
    assert ("shared+bias" in d) == (with_s or with_b)
    if in_place:
        assert out.data_ptr() == out_buf.data_ptr()

    # the same steps one by one
    r = moe.route(c.x, c.wg, k, bias=c.bias, want_p=False, quant=a8, n_group=G or None, topk_group=TG or None)
    wdt = {"bf16": torch.bfloat16, "i8": torch.int8, "i4": torch.uint8, "i4a8": "w4a8"}[s.w_dtype]
    bm = moe.ffn_block_m(T, H, s.I, s.E, k, wdt)
    a = moe.align(r["ids"], s.E, c.C or 0, bm)
    y = moe.expert_ffn(r["xq"] if a8 else c.x, c.w13, c.w2, a["sorted_slot"], a["tiles"], a["num_tiles"], bm, k,
                       topk_w=r["w"], xs=r["xs"], s13=c.s13, s2=c.s2, w4a8=w4a8)
    ref_d = moe.combine_shared(y, a["pos"], None, T, k, torch.bfloat16, shared=S_d, shared_factor=f, bias=b_d)
    torch.cuda.synchronize()
    assert torch.equal(aux["topk_ids"], r["ids"])
    assert torch.equal(out.view(torch.int16), ref_d.view(torch.int16))

    # against the oracle
    S64 = moe_synth.bf16_bits_as_f32(S).astype(np.float64) if with_s else None
    ro = oracle.layer(c.inp.x, s.x_dtype, c.inp.wg, s.wg_dtype, c.inp.bias, c.inp.w13, c.inp.w2, s.w_dtype, k,
                      s.capacity_factor, c.inp.s13, c.inp.s2, n_group=G, topk_group=TG, shared=S64,
                      shared_factor=f, out_bias=b)
    rr = ro["route"]
    band = dict(rr, gap_p=np.minimum(rr["gap_p"], rr["gap_group"])) if G else rr
    same = check_ids(aux["topk_ids"].cpu().numpy(), band)
    pos_g = aux["pos"].cpu().numpy()
    agree = same & ((pos_g >= 0) == (ro["align"]["pos"].reshape(T, k) >= 0)).all(axis=1)
    assert agree.mean() > 0.97
    got = out.float().cpu().numpy().astype(np.float64)
    rel = _rel(got[agree], ro["out"][agree])
    print(f"[layer_ex] {s.name}: rel-L2 {rel:.3e} over {int(agree.sum())}/{T} tokens")
    assert rel <= TOL[s.w_dtype], rel
