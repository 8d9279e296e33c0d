"""ctypes binding of ``libmoe.so`` (argument marshalling only).

Every function here passes device pointers, sizes and the current HIP stream
to the C ABI declared in ``include/moe.h``; all computation happens in the
HIP kernels.  PyTorch provides device memory (outputs and workspaces) and the
stream.  A missing library raises at import: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_I8, MOE_I4, MOE_I4A8 = 0, 1, 2, 3, 4
# torch.uint8 expert weights are int4 codes packed by pack_int4: W4A16, or
# W4A8 where a call says so (w4a8=True, or the weight dtype given as "w4a8")
_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.int8: MOE_I8, torch.uint8: MOE_I4, "w4a8": MOE_I4A8}


def _wdt(w: torch.Tensor, w4a8: bool) -> int:
    if w4a8:
        if w.dtype != torch.uint8:
            raise ValueError("W4A8 takes packed int4 weights (uint8, from pack_int4)")
        return MOE_I4A8
    return _DT[w.dtype]

_vp, _i32, _i64, _sz, _f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double
_st = ctypes.c_int

# name -> (restype, argtypes); the same names and order as include/moe.h
SIGNATURES = {
    "moe_route_workspace_size": (_sz, [_i64, _i32, _i32, _i32]),
    "moe_route": (_st, [_vp, _i32, _vp, _i32, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                        _vp, _sz, _vp]),
    "moe_route_grouped": (_st, [_vp, _i32, _vp, _i32, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                _vp, _vp, _vp, _sz, _vp]),
    "moe_capacity": (_i64, [_i64, _i32, _i32, _f64]),
    "moe_align_workspace_size": (_sz, [_i64, _i32, _i32]),
    "moe_align_max_tiles": (_i64, [_i64, _i32, _i32, _i32]),
    "moe_align": (_st, [_vp, _i64, _i32, _i32, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                        _sz, _vp]),
    "moe_ffn_block_m": (_i32, [_i64, _i32, _i32, _i32, _i32, _i32]),
    "moe_ffn_workspace_size": (_sz, [_i64, _i32, _i32, _i32, _i32, _i32]),
    "moe_expert_ffn": (_st, [_vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                             _i64, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _sz, _vp]),
    "moe_ffn_up": (_st, [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32,
                         _i32, _vp, _sz, _vp]),
    "moe_ffn_down": (_st, [_vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i64, _i32, _i32, _i32, _i32, _vp,
                           _i32, _vp, _sz, _vp]),
    "moe_pack_int4": (_st, [_vp, _i64, _i32, _vp, _vp]),
    "moe_route_align_workspace_size": (_sz, [_i64, _i32, _i32, _i32]),
    "moe_route_align": (_st, [_vp, _i32, _vp, _i32, _vp, _i64, _i32, _i32, _i32, _i64, _i32, _vp, _vp, _vp, _vp, _vp,
                              _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_combine": (_st, [_vp, _i32, _vp, _vp, _i64, _i32, _i32, _vp, _i32, _vp]),
    "moe_combine_shared": (_st, [_vp, _i32, _vp, _vp, _i64, _i32, _i32, _vp, ctypes.c_float, _vp, _vp,
                                 _i32, _vp]),
    "moe_layer_workspace_size": (_sz, [_i64, _i32, _i32, _i32, _i32, _i32, _i32]),
    "moe_layer": (_st, [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _i64, _i32, _i32, _i32,
                        _i32, _i64, _vp, _i32, _vp, _vp, _sz, _vp]),
    "moe_layer_ex": (_st, [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _i64, _i32, _i32, _i32,
                           _i32, _i64, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "moe_layer_noalloc": (_st, [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _i64, _i32, _i32, _i32,
                                _i32, _i64, _vp, _i32, _vp, _vp]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_last_dispatch": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_char_p, []),
}


class MoeLayerAux(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("topk_ids", "topk_w", "topk_p", "counts", "offsets", "sorted_slot",
                                   "pos", "num_dropped", "xq", "xs")] + [("stage_events", _vp * 6)]


class MoeLayerOptions(ctypes.Structure):
    _fields_ = [("n_group", _i32), ("topk_group", _i32), ("shared", _vp), ("shared_factor", ctypes.c_float),
                ("out_bias", _vp)]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"moe status {status}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run routing_dispatch_expert_gate_amd.build.build() "
                          "(hipcc, gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib.moe_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ws(nbytes: int, device) -> torch.Tensor | None:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device) if nbytes else None


def last_dispatch() -> str:
    return lib.moe_last_dispatch().decode()


def version() -> str:
    return lib.moe_version().decode()


def capacity(T: int, k: int, E: int, factor: float) -> int:
    return int(lib.moe_capacity(T, k, E, float(factor)))


def route(x: torch.Tensor, wg: torch.Tensor, k: int, bias: torch.Tensor | None = None,
          want_p: bool = True, quant: bool = False, n_group: int | None = None,
          topk_group: int | None = None) -> dict:
    """moe_route: returns ids [T,k] int32, w [T,k] fp32, p [T,k] fp32 (or None),
    and xq [T,H] int8 / xs [T] fp32 when ``quant``.  With ``n_group`` and
    ``topk_group`` it calls moe_route_grouped (group-limited selection)."""
    _dev(x, "x"), _dev(wg, "wg")
    T, H = x.shape
    E = wg.shape[0]
    dev = x.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    p = torch.empty((T, k), dtype=torch.float32, device=dev) if want_p else None
    xq = torch.empty((T, H), dtype=torch.int8, device=dev) if quant else None
    xs = torch.empty((T,), dtype=torch.float32, device=dev) if quant else None
    if bias is not None:
        _dev(bias, "bias")
    nws = lib.moe_route_workspace_size(T, H, E, k)
    ws = _ws(nws, dev)
    if (n_group is None) != (topk_group is None):
        raise ValueError("n_group and topk_group go together")
    if n_group is None:
        _check(lib.moe_route(_p(x), _DT[x.dtype], _p(wg), _DT[wg.dtype], _p(bias), T, H, E, k, _p(ids),
                             _p(w), _p(p), _p(xq), _p(xs), _p(ws), nws, _stream(dev)))
    else:
        _check(lib.moe_route_grouped(_p(x), _DT[x.dtype], _p(wg), _DT[wg.dtype], _p(bias), T, H, E, k,
                                     int(n_group), int(topk_group), _p(ids), _p(w), _p(p), _p(xq), _p(xs),
                                     _p(ws), nws, _stream(dev)))
    return {"ids": ids, "w": w, "p": p, "xq": xq, "xs": xs}


def route_align(x: torch.Tensor, wg: torch.Tensor, k: int, capacity: int = 0, block_m: int = 128,
                bias: torch.Tensor | None = None, want_p: bool = True, quant: bool = False) -> dict:
    """moe_route_align: the outputs of route() and align() from one call."""
    _dev(x, "x"), _dev(wg, "wg")
    T, H = x.shape
    E = wg.shape[0]
    dev = x.device
    n = T * k
    mt = int(lib.moe_align_max_tiles(T, k, E, block_m))
    i32 = torch.int32
    o = {
        "ids": torch.empty((T, k), dtype=i32, device=dev), "w": torch.empty((T, k), dtype=torch.float32, device=dev),
        "p": torch.empty((T, k), dtype=torch.float32, device=dev) if want_p else None,
        "xq": torch.empty((T, H), dtype=torch.int8, device=dev) if quant else None,
        "xs": torch.empty((T,), dtype=torch.float32, device=dev) if quant else None,
        "counts": torch.empty(E, dtype=i32, device=dev), "offsets": torch.empty(E + 1, dtype=i32, device=dev),
        "sorted_slot": torch.empty(n, dtype=i32, device=dev), "pos": torch.empty((T, k), dtype=i32, device=dev),
        "tiles": torch.empty((max(mt, 1), 4), dtype=i32, device=dev), "num_tiles": torch.empty(1, dtype=i32, device=dev),
        "num_dropped": torch.empty(1, dtype=i32, device=dev),
    }
    if bias is not None:
        _dev(bias, "bias")
    nws = lib.moe_route_align_workspace_size(T, H, E, k)
    ws = _ws(nws, dev)
    _check(lib.moe_route_align(_p(x), _DT[x.dtype], _p(wg), _DT[wg.dtype], _p(bias), T, H, E, k, int(capacity),
                               block_m, _p(o["ids"]), _p(o["w"]), _p(o["p"]), _p(o["xq"]), _p(o["xs"]),
                               _p(o["counts"]), _p(o["offsets"]), _p(o["sorted_slot"]), _p(o["pos"]),
                               _p(o["tiles"]), _p(o["num_tiles"]), _p(o["num_dropped"]), _p(ws), nws,
                               _stream(dev)))
    return o


def align(ids: torch.Tensor, E: int, capacity: int = 0, block_m: int = 128) -> dict:
    """moe_align on device ids [T,k]."""
    _dev(ids, "ids")
    T, k = ids.shape
    dev = ids.device
    n = T * k
    mt = int(lib.moe_align_max_tiles(T, k, E, block_m))
    out = {
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "sorted_slot": torch.empty(n, dtype=torch.int32, device=dev),
        "pos": torch.empty((T, k), dtype=torch.int32, device=dev),
        "tiles": torch.empty((max(mt, 1), 4), dtype=torch.int32, device=dev),
        "num_tiles": torch.empty(1, dtype=torch.int32, device=dev),
        "num_dropped": torch.empty(1, dtype=torch.int32, device=dev),
    }
    nws = lib.moe_align_workspace_size(T, k, E)
    ws = _ws(nws, dev)
    _check(lib.moe_align(_p(ids), T, k, E, int(capacity), block_m, _p(out["counts"]), _p(out["offsets"]),
                         _p(out["sorted_slot"]), _p(out["pos"]), _p(out["tiles"]), _p(out["num_tiles"]),
                         _p(out["num_dropped"]), _p(ws), nws, _stream(dev)))
    return out


def _inner(w: torch.Tensor) -> int:
    """K extent of a weight tensor's rows (packed int4 holds two per byte)."""
    return w.shape[-1] * (2 if w.dtype == torch.uint8 else 1)


def pack_int4(codes: torch.Tensor) -> torch.Tensor:
    """moe_pack_int4: int8 codes [..., K] in [-8, 7] -> packed uint8 [..., K/2]."""
    _dev(codes, "codes")
    if codes.dtype != torch.int8:
        raise ValueError("codes must be int8")
    K = codes.shape[-1]
    rows = codes.numel() // K if K else 0
    out = torch.empty(codes.shape[:-1] + (K // 2,), dtype=torch.uint8, device=codes.device)
    _check(lib.moe_pack_int4(_p(codes), rows, K, _p(out), _stream(codes.device)))
    return out


def ffn_block_m(T: int, H: int, I: int, E: int, k: int, w_dtype) -> int:
    return int(lib.moe_ffn_block_m(T, H, I, E, k, _DT[w_dtype]))


def expert_ffn(x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, sorted_slot: torch.Tensor,
               tiles: torch.Tensor, num_tiles: torch.Tensor, block_m: int, k: int,
               topk_w: torch.Tensor | None = None, xs: torch.Tensor | None = None,
               s13: torch.Tensor | None = None, s2: torch.Tensor | None = None,
               w4a8: bool = False) -> torch.Tensor:
    """moe_expert_ffn: returns y_sorted [T*k, H] (rows >= N unwritten).
    Packed int4 weights run W4A16 with bf16 x, or W4A8 with ``w4a8`` (x = int8
    codes, xs their scales)."""
    for t, nme in ((x, "x"), (w13, "w13"), (w2, "w2"), (sorted_slot, "sorted_slot"), (tiles, "tiles")):
        _dev(t, nme)
    T, H = x.shape
    E, I = w2.shape[0], _inner(w2)
    dev = x.device
    ydt = torch.float32 if w13.dtype == torch.float32 else torch.bfloat16
    y = torch.empty((T * k, H), dtype=ydt, device=dev)
    wd = _wdt(w13, w4a8)
    nws = lib.moe_ffn_workspace_size(T, H, I, E, k, wd)
    ws = _ws(nws, dev)
    _check(lib.moe_expert_ffn(_p(x), _DT[x.dtype], _p(xs), _p(w13), _p(w2), wd, _p(s13), _p(s2),
                              _p(sorted_slot), _p(tiles), _p(num_tiles), block_m, _p(topk_w), T, H, I, E, k,
                              _p(y), _DT[ydt], _p(ws), nws, _stream(dev)))
    return y


def ffn_workspace(T: int, H: int, I: int, E: int, k: int, w_dtype: torch.dtype, device="cuda"):
    """A workspace for moe_ffn_up / moe_ffn_down (it carries h between them)."""
    n = int(lib.moe_ffn_workspace_size(T, H, I, E, k, _DT[w_dtype]))
    return _ws(n, device), n


def ffn_up(x, w13, sorted_slot, tiles, num_tiles, block_m, k, E, I, ws, xs=None, s13=None, w4a8=False):
    """moe_ffn_up into the workspace ``ws`` = (tensor, nbytes) from ffn_workspace."""
    T, H = x.shape
    _check(lib.moe_ffn_up(_p(x), _DT[x.dtype], _p(xs), _p(w13), _wdt(w13, w4a8), _p(s13), _p(sorted_slot),
                          _p(tiles), _p(num_tiles), block_m, T, H, I, E, k, _p(ws[0]), ws[1],
                          _stream(x.device)))


def ffn_down(w2, sorted_slot, tiles, num_tiles, block_m, k, T, ws, y, topk_w=None, s2=None, w4a8=False):
    """moe_ffn_down from the workspace filled by ffn_up into ``y`` [T*k, H]."""
    E, H, I = w2.shape[0], w2.shape[1], _inner(w2)
    _check(lib.moe_ffn_down(_p(w2), _wdt(w2, w4a8), _p(s2), _p(sorted_slot), _p(tiles), _p(num_tiles),
                            block_m, _p(topk_w), T, H, I, E, k, _p(y), _DT[y.dtype], _p(ws[0]), ws[1],
                            _stream(y.device)))


def combine(y_sorted: torch.Tensor, pos: torch.Tensor, topk_w: torch.Tensor | None, T: int, k: int,
            out_dtype: torch.dtype) -> torch.Tensor:
    """moe_combine: out [T, H]."""
    _dev(y_sorted, "y_sorted"), _dev(pos, "pos")
    H = y_sorted.shape[1]
    out = torch.empty((T, H), dtype=out_dtype, device=y_sorted.device)
    _check(lib.moe_combine(_p(y_sorted), _DT[y_sorted.dtype], _p(pos), _p(topk_w), T, k, H, _p(out),
                           _DT[out_dtype], _stream(y_sorted.device)))
    return out


def combine_shared(y_sorted: torch.Tensor, pos: torch.Tensor, topk_w: torch.Tensor | None, T: int, k: int,
                   out_dtype: torch.dtype, shared: torch.Tensor | None = None, shared_factor: float = 1.0,
                   bias: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """moe_combine_shared: out [T, H] = routed sum + shared_factor * shared + bias.
    `out` may be `shared` itself (in-place update of the shared expert's output)."""
    _dev(y_sorted, "y_sorted"), _dev(pos, "pos")
    H = y_sorted.shape[1]
    if shared is not None:
        _dev(shared, "shared")
        if shared.dtype != out_dtype or tuple(shared.shape) != (T, H):
            raise ValueError(f"shared must be [{T}, {H}] {out_dtype}")
    if bias is not None:
        _dev(bias, "bias")
        if bias.dtype != torch.float32 or tuple(bias.shape) != (H,):
            raise ValueError(f"bias must be [{H}] float32")
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y_sorted.device)
    _check(lib.moe_combine_shared(_p(y_sorted), _DT[y_sorted.dtype], _p(pos), _p(topk_w), T, k, H,
                                  _p(shared), float(shared_factor), _p(bias), _p(out), _DT[out_dtype],
                                  _stream(y_sorted.device)))
    return out


class Layer:
    """moe_layer with a workspace allocated once and re-used across calls."""

    def __init__(self, T: int, H: int, I: int, E: int, k: int, x_dtype: torch.dtype,
                 w_dtype, device="cuda"):
        self.shape = (T, H, I, E, k)
        self.x_dtype, self.w_dtype = x_dtype, w_dtype
        self.nws = lib.moe_layer_workspace_size(T, H, I, E, k, _DT[x_dtype], _DT[w_dtype])
        self.ws = _ws(self.nws, device)

    def __call__(self, x, wg, w13, w2, capacity=0, bias=None, s13=None, s2=None, out=None, aux=None,
                 options: dict | None = None):
        """``options`` (a dict of moe_layer_options members: n_group,
        topk_group, shared, shared_factor, out_bias) selects moe_layer_ex.
        ``aux`` maps moe_layer_aux member names to device tensors, and
        ``stage_events`` to six hipEvent_t handles (ints, or None)."""
        T, H, I, E, k = self.shape
        if out is None:
            out = torch.empty((T, H), dtype=x.dtype, device=x.device)
        aux_s = None
        if aux is not None:
            aux_s = MoeLayerAux(**{n: (aux[n].data_ptr() if aux.get(n) is not None else None)
                                   for n, _ in MoeLayerAux._fields_ if n != "stage_events"})
            ev = aux.get("stage_events")
            if ev is not None:
                if len(ev) != 6:
                    raise ValueError("stage_events takes six hipEvent_t handles (ints or None)")
                aux_s.stage_events = (_vp * 6)(*ev)
        args = [_p(x), _DT[x.dtype], _p(wg), _DT[wg.dtype], _p(bias), _p(w13), _p(w2), _DT[self.w_dtype],
                _p(s13), _p(s2), T, H, I, E, k, int(capacity), _p(out), _DT[out.dtype],
                ctypes.byref(aux_s) if aux_s is not None else None]
        if options is None:
            _check(lib.moe_layer(*args, _p(self.ws), self.nws, _stream(x.device)))
            return out
        o = dict(options)
        sh, ob = o.get("shared"), o.get("out_bias")
        if sh is not None:
            _dev(sh, "shared")
            if sh.dtype != out.dtype or tuple(sh.shape) != (T, H):
                raise ValueError(f"shared must be [{T}, {H}] {out.dtype}")
        if ob is not None:
            _dev(ob, "out_bias")
            if ob.dtype != torch.float32 or tuple(ob.shape) != (H,):
                raise ValueError(f"out_bias must be [{H}] float32")
        opt = MoeLayerOptions(int(o.get("n_group", 0)), int(o.get("topk_group", 0)), _p(sh),
                              float(o.get("shared_factor", 1.0)), _p(ob))
        _check(lib.moe_layer_ex(*args, ctypes.byref(opt), _p(self.ws), self.nws, _stream(x.device)))
        return out


def layer(x, wg, w13, w2, k, capacity=0, bias=None, s13=None, s2=None, aux=None, w4a8=False, options=None):
    """One moe_layer call (allocates its workspace); ``aux`` maps moe_layer_aux
    member names to device tensors that receive the intermediates; ``w4a8``
    runs packed int4 weights with int8 activations; ``options`` (dict of
    moe_layer_options members) calls moe_layer_ex."""
    T, H = x.shape
    E, I = w2.shape[0], _inner(w2)
    _wdt(w13, w4a8)
    wd = "w4a8" if w4a8 else w13.dtype
    return Layer(T, H, I, E, k, x.dtype, wd, x.device)(x, wg, w13, w2, capacity, bias, s13, s2, aux=aux,
                                                         options=options)
