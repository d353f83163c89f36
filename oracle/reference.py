"""Python driver for the C oracle (moe_oracle.c): the layer forward, stage by stage.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may use this module; the product package must
never import it.

The steps follow the MoE layer as the pages describe it (MegaMoE post, "The
problem": route to a top-K subset of experts, quantize activations, two grouped
GEMMs, combine; FlashInfer PR #4366, "Description": router weight on the output
side, sum_r p_r W2_r(a_r), or on the input side, sum_r W2_r(p_r a_r), the latter
scaled in FP32 after the activation and before the FC2-input quantization or
BF16 store):

  S1 route -> S2 permute -> S3 quantize x -> S4 FC1 -> S5 activation, placement,
  FC2-input precision -> S6 FC2 -> S7 finalize (fixed k order, fp64).

Each stage is one C call (or a loop of them); Python only moves arrays between
stages. Work over routes may be spread over threads (``threads``): the C calls
release the GIL, each route's arithmetic is unchanged, and reductions across
routes (the per-tensor amax, the finalize) are done after all routes finish, so
the result does not depend on the thread count.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "moe_oracle.c")

FMT_NVFP4, FMT_MXFP8, FMT_MXFP4 = 0, 1, 2
ACT_SWIGLU, ACT_RELU2 = 0, 1
MODES = ("w4a4_tensor", "w4a4_token", "w4a16", "mxfp8", "w4a4_token_4o6", "w4a4_token_mxfp4")
# modes whose activations carry one NVFP4 global scale per row (token / route)
PER_ROW_MODES = ("w4a4_token", "w4a4_token_4o6", "w4a4_token_mxfp4")


def weight_format(mode: str) -> str:
    """The prepared-weight format a mode consumes."""
    return {"mxfp8": "mxfp8", "w4a4_token_mxfp4": "mxfp4"}.get(mode, "nvfp4")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC",
             "-shared", "-o", _SO, _SRC, "-lm"])
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        d, i, f, u16 = ctypes.c_double, ctypes.c_int, ctypes.c_float, ctypes.c_uint16
        P = ctypes.c_void_p
        L.orc_e2m1_decode.restype = d; L.orc_e2m1_decode.argtypes = [i]
        L.orc_e2m1_encode.restype = i; L.orc_e2m1_encode.argtypes = [d]
        L.orc_e4m3_decode.restype = d; L.orc_e4m3_decode.argtypes = [i]
        L.orc_e4m3_encode.restype = i; L.orc_e4m3_encode.argtypes = [d]
        L.orc_e8m0_decode.restype = d; L.orc_e8m0_decode.argtypes = [i]
        L.orc_bf16_to_f32.restype = f; L.orc_bf16_to_f32.argtypes = [u16]
        L.orc_f32_to_bf16.restype = u16; L.orc_f32_to_bf16.argtypes = [f]
        L.orc_route.restype = None; L.orc_route.argtypes = [i, i, i, P, P, P]
        L.orc_permute.restype = None; L.orc_permute.argtypes = [i, i, i, P, P, P, P, P]
        L.orc_absmax.restype = f; L.orc_absmax.argtypes = [P, ctypes.c_size_t]
        L.orc_nvfp4_global_scale.restype = f; L.orc_nvfp4_global_scale.argtypes = [f]
        L.orc_nvfp4_quantize.restype = None; L.orc_nvfp4_quantize.argtypes = [i, P, f, P, P]
        L.orc_nvfp4_global_scale_4o6.restype = f; L.orc_nvfp4_global_scale_4o6.argtypes = [f]
        L.orc_nvfp4_quantize_4o6.restype = None; L.orc_nvfp4_quantize_4o6.argtypes = [i, P, f, P, P]
        L.orc_nvfp4_dequant.restype = None; L.orc_nvfp4_dequant.argtypes = [i, P, P, f, P]
        L.orc_mxfp4_reblock.restype = None; L.orc_mxfp4_reblock.argtypes = [i, P, P, P, P]
        L.orc_mxfp4_dequant.restype = None; L.orc_mxfp4_dequant.argtypes = [i, P, P, P]
        L.orc_mxfp8_quantize.restype = None; L.orc_mxfp8_quantize.argtypes = [i, P, P, P]
        L.orc_mxfp8_dequant.restype = None; L.orc_mxfp8_dequant.argtypes = [i, P, P, P]
        L.orc_quantize_weight.restype = None
        L.orc_quantize_weight.argtypes = [i, i, i, P, P, P, P]
        L.orc_expert_matvec.restype = None
        L.orc_expert_matvec.argtypes = [i, i, i, P, P, f, P, P]
        L.orc_expert_matvec_rows.restype = None
        L.orc_expert_matvec_rows.argtypes = [i, i, P, P, f, P, i, P, P]
        L.orc_activation.restype = None; L.orc_activation.argtypes = [i, i, P, i, d, i, P]
        L.orc_finalize.restype = None; L.orc_finalize.argtypes = [i, i, i, P, P, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _pmap(fn, items, threads):
    items = list(items)
    if threads <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


# --------------------------------------------------------------------------
# codecs (scalar)
# --------------------------------------------------------------------------

def e2m1_decode(c): return lib().orc_e2m1_decode(int(c))
def e2m1_encode(u): return lib().orc_e2m1_encode(float(u))
def e4m3_decode(c): return lib().orc_e4m3_decode(int(c))
def e4m3_encode(u): return lib().orc_e4m3_encode(float(u))
def e8m0_decode(c): return lib().orc_e8m0_decode(int(c))


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    L = lib()
    return np.array([L.orc_f32_to_bf16(float(x)) for x in v], dtype=np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# S1 / S2
# --------------------------------------------------------------------------

def route(logits: np.ndarray, K: int):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, K), np.int32)
    p = np.empty((T, K), np.float64)
    lib().orc_route(T, E, K, _p(logits), _p(ids), _p(p))
    return ids, p


def permute(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    R = T * K
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    r2r = np.empty(R, np.int32)
    rt2row = np.empty(R, np.int32)
    lib().orc_permute(T, K, E, _p(ids), _p(counts), _p(offsets), _p(r2r), _p(rt2row))
    return counts, offsets, r2r, rt2row


# --------------------------------------------------------------------------
# quantizers over [rows, n] fp32 matrices
# --------------------------------------------------------------------------

def absmax(v: np.ndarray) -> np.float32:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return np.float32(lib().orc_absmax(_p(v), v.size))


def nvfp4_quantize(v: np.ndarray, per_row: bool, threads: int = 1, four_over_six: bool = False):
    """NVFP4 of a [rows, n] fp32 matrix; one global scale for the whole matrix
    (per_row=False) or one per row. four_over_six: the 4-over-6 block choice
    (orc_nvfp4_quantize_4o6, one global scale per row only). Returns unpacked
    codes [rows, n] u8, block scales [rows, n/16] u8 (E4M3 bits) and g ([1] or
    [rows]) fp32."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, n = v.shape
    L = lib()
    codes = np.empty((rows, n), np.uint8)
    sf = np.empty((rows, n // 16), np.uint8)
    assert per_row or not four_over_six, "4-over-6 is a per-token contract"
    gscale = L.orc_nvfp4_global_scale_4o6 if four_over_six else L.orc_nvfp4_global_scale
    quant = L.orc_nvfp4_quantize_4o6 if four_over_six else L.orc_nvfp4_quantize
    if per_row:
        g = np.array([gscale(absmax(v[r])) for r in range(rows)], np.float32)
    else:
        g = np.array([gscale(absmax(v))], np.float32)

    def one(r):
        gr = float(g[r] if per_row else g[0])
        quant(n, _p(v[r]), gr, _p(codes[r]), _p(sf[r]))
    _pmap(one, range(rows), threads)
    return codes, sf, g


def nvfp4_dequant(codes, sf, g, per_row: bool) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sf = np.ascontiguousarray(sf, dtype=np.uint8)
    rows, n = codes.shape
    out = np.empty((rows, n), np.float64)
    L = lib()
    for r in range(rows):
        gr = float(g[r] if per_row else g[0])
        L.orc_nvfp4_dequant(n, _p(codes[r]), _p(sf[r]), gr, _p(out[r]))
    return out


def mxfp4_reblock(codes: np.ndarray, sf: np.ndarray, threads: int = 1):
    """NVFP4 rows (unpacked codes [rows, n], E4M3 scales [rows, n/16]) re-blocked
    to MXFP4 (E2M1 codes [rows, n], E8M0 scales [rows, n/32]) by
    orc_mxfp4_reblock; the global scales are not involved."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sf = np.ascontiguousarray(sf, dtype=np.uint8)
    rows, n = codes.shape
    mc = np.empty((rows, n), np.uint8)
    ms = np.empty((rows, n // 32), np.uint8)
    L = lib()

    def one(r):
        L.orc_mxfp4_reblock(n, _p(codes[r]), _p(sf[r]), _p(mc[r]), _p(ms[r]))
    _pmap(one, range(rows), threads)
    return mc, ms


def mxfp4_dequant(codes, sc, g=None, per_row: bool = True) -> np.ndarray:
    """E2M1(code) * 2^X (* g per row or for all rows), fp64 (exact)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    rows, n = codes.shape
    out = np.empty((rows, n), np.float64)
    L = lib()
    for r in range(rows):
        L.orc_mxfp4_dequant(n, _p(codes[r]), _p(sc[r]), _p(out[r]))
        if g is not None:
            out[r] *= float(g[r] if per_row else g[0])
    return out


def mxfp8_quantize(v: np.ndarray, threads: int = 1):
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, n = v.shape
    codes = np.empty((rows, n), np.uint8)
    sc = np.empty((rows, n // 32), np.uint8)
    L = lib()

    def one(r):
        L.orc_mxfp8_quantize(n, _p(v[r]), _p(codes[r]), _p(sc[r]))
    _pmap(one, range(rows), threads)
    return codes, sc


def mxfp8_dequant(codes, sc) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    rows, n = codes.shape
    out = np.empty((rows, n), np.float64)
    L = lib()
    for r in range(rows):
        L.orc_mxfp8_dequant(n, _p(codes[r]), _p(sc[r]), _p(out[r]))
    return out


# --------------------------------------------------------------------------
# S0: expert weights, quantized per expert on demand
# --------------------------------------------------------------------------

class QuantWeights:
    """Quantized expert weights held by the oracle (codes unpacked, one byte per
    element). ``provider(e)`` returns expert e's fp32 (W1 [N1, H], W2 [H, I]) in
    the checkpoint [N, K] layout; experts are quantized the first time they
    are needed."""

    def __init__(self, fmt: str, E: int, H: int, I: int, act: str, provider):
        # "mxfp4": NVFP4 quantization (per-expert global scale), then each row
        # re-blocked to MXFP4 (orc_mxfp4_reblock); the global scale is kept
        self.fmt = {"mxfp8": FMT_MXFP8, "mxfp4": FMT_MXFP4}.get(fmt, FMT_NVFP4)
        self.E, self.H, self.I = E, H, I
        self.N1 = 2 * I if act == "swiglu" else I
        self.provider = provider
        self.q = {}

    def _quant(self, N, K, w):
        w = np.ascontiguousarray(w, dtype=np.float32)
        assert w.shape == (N, K)
        codes = np.empty((N, K), np.uint8)
        blk = 32 if self.fmt == FMT_MXFP8 else 16
        sc = np.empty((N, K // blk), np.uint8)
        g = ctypes.c_float(0.0)
        qfmt = FMT_MXFP8 if self.fmt == FMT_MXFP8 else FMT_NVFP4
        lib().orc_quantize_weight(qfmt, N, K, _p(w), _p(codes), _p(sc), ctypes.byref(g))
        if self.fmt == FMT_MXFP4:
            codes, sc = mxfp4_reblock(codes, sc)
        return codes, sc, np.float32(g.value)

    def ensure(self, experts, threads: int = 1):
        todo = sorted(set(int(e) for e in experts) - set(self.q))

        def one(e):
            w1, w2 = self.provider(e)
            return e, self._quant(self.N1, self.H, w1), self._quant(self.H, self.I, w2)
        for e, q1, q2 in _pmap(one, todo, threads):
            self.q[e] = (q1, q2)

    def fc1(self, e, a: np.ndarray) -> np.ndarray:
        (c, s, g), _ = self.q[e]
        out = np.empty(self.N1, np.float64)
        lib().orc_expert_matvec(self.fmt, self.N1, self.H, _p(c), _p(s), float(g), _p(a), _p(out))
        return out

    def fc2(self, e, a: np.ndarray) -> np.ndarray:
        _, (c, s, g) = self.q[e]
        out = np.empty(self.H, np.float64)
        lib().orc_expert_matvec(self.fmt, self.H, self.I, _p(c), _p(s), float(g), _p(a), _p(out))
        return out

    def dequant_matrix(self, e, which: int) -> np.ndarray:
        """Dense fp64 dequantized W1 [N1, H] (which = 0) or W2 [H, I] (which = 1)
        of expert e, each element decoded by the oracle's own codec (exact)."""
        c, s, g = self.q[e][which]
        N = c.shape[0]
        if self.fmt == FMT_NVFP4:
            return nvfp4_dequant(c, s, np.array([g] * N, np.float32), per_row=True)
        if self.fmt == FMT_MXFP4:
            return mxfp4_dequant(c, s, np.array([g], np.float32), per_row=False)
        return mxfp8_dequant(c, s)

    def dequant(self, e):
        """Dense fp64 dequantized (W1 [N1, H], W2 [H, I]) of expert e."""
        return [self.dequant_matrix(e, 0), self.dequant_matrix(e, 1)]

    def fc1_rows(self, e, A: np.ndarray) -> np.ndarray:
        """FC1 of several fp64 input rows A [n, H] for expert e: one fp64 matrix
        product with the dequantized W1 (the grouped GEMM by its definition; the
        library matmul only changes the fp64 summation order)."""
        return np.ascontiguousarray(A, dtype=np.float64) @ self.dequant_matrix(e, 0).T

    def fc2_rows(self, e, A: np.ndarray) -> np.ndarray:
        """FC2 of several fp64 input rows A [n, I] for expert e (as fc1_rows)."""
        return np.ascontiguousarray(A, dtype=np.float64) @ self.dequant_matrix(e, 1).T


# --------------------------------------------------------------------------
# S3: FC1-input quantization (in token order; FC1 gathers rows)
# --------------------------------------------------------------------------

def quantize_x(x_bits: np.ndarray, mode: str, threads: int = 1) -> dict:
    """x_bits: [T, H] bf16 bit patterns. Returns the quantized views and a
    function deq(t) giving the fp64 FC1 input row of token t."""
    x = bf16_bits_to_f32(x_bits).reshape(x_bits.shape)
    if mode == "w4a16":
        return {"deq": lambda t: x[t].astype(np.float64)}
    if mode == "mxfp8":
        codes, sc = mxfp8_quantize(x, threads)
        return {"codes": codes, "scales": sc,
                "deq": lambda t: mxfp8_dequant(codes[t:t + 1], sc[t:t + 1])[0]}
    per_row = mode in PER_ROW_MODES
    codes, sf, g = nvfp4_quantize(x, per_row, threads, four_over_six=mode == "w4a4_token_4o6")
    if mode == "w4a4_token_mxfp4":
        mc, ms = mxfp4_reblock(codes, sf, threads)
        return {"codes": codes, "scales": sf, "g": g, "mx_codes": mc, "mx_scales": ms,
                "deq": lambda t: mxfp4_dequant(mc[t:t + 1], ms[t:t + 1], g[t:t + 1])[0]}
    return {"codes": codes, "scales": sf, "g": g,
            "deq": lambda t: nvfp4_dequant(codes[t:t + 1], sf[t:t + 1],
                                           g[t:t + 1] if per_row else g, per_row)[0]}


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------

def _blas_single_thread():
    """Context that keeps BLAS to one thread inside the oracle's own thread pool
    (each worker runs its own matrix product)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1, user_api="blas")
    except ImportError:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


def _by_expert(routes, ids):
    """{expert: [routes in ascending order]} for the given routes."""
    groups = {}
    for r in routes:
        groups.setdefault(int(ids.flat[r]), []).append(int(r))
    return groups


def fc2_finalize(W: QuantWeights, ids: np.ndarray, p: np.ndarray, K: int, on_input: bool,
                 tokens, a2_of_route, threads: int = 1, batched: bool = False):
    """S6 + S7 for the given tokens: o_r = W2_{e(r)} a2_r for every route r of
    those tokens (fp64), then y[t] = sum_{k<K} w_{t,k} o_{tK+k} in fixed k order
    (fp64), w = p for output-side placement and 1 for input-side placement
    (neutral finalize weights, FlashInfer PR #4366, "Description").

    a2_of_route(r) gives route r's fp64 FC2 input row (the dequantized FC2
    input). Returns (o [len(tokens)*K, H] in route order, y [len(tokens), H])."""
    toks = [int(t) for t in tokens]
    want = [t * K + k for t in toks for k in range(K)]
    H = W.H
    if not want:
        return np.zeros((0, H)), np.zeros((0, H))
    if batched:
        groups = _by_expert(want, ids)

        def one(item):
            e, rs = item
            return rs, W.fc2_rows(e, np.stack([a2_of_route(r) for r in rs]))
        pos = {r: i for i, r in enumerate(want)}
        o = np.empty((len(want), H), np.float64)
        with _blas_single_thread() if threads > 1 else _nullctx():
            for rs, block in _pmap(one, sorted(groups.items()), threads):
                o[[pos[r] for r in rs]] = block
    else:
        o = np.stack(_pmap(lambda r: W.fc2(int(ids.flat[r]), np.ascontiguousarray(a2_of_route(r))),
                           want, threads))
    # S7: finalize in fixed k order; unit weights for input-side placement
    w = None if on_input else np.ascontiguousarray(p[toks], dtype=np.float64)
    y = np.empty((len(toks), H), np.float64)
    lib().orc_finalize(len(toks), K, H, _p(np.ascontiguousarray(o)),
                       _p(np.arange(len(want), dtype=np.int32)),
                       _p(w) if w is not None else None, _p(y))
    return o, y


def _nullctx():
    import contextlib
    return contextlib.nullcontext()


def forward(x_bits: np.ndarray, logits: np.ndarray, W: QuantWeights, K: int, mode: str,
            act: str, on_input: bool, tokens=None, threads: int = 1,
            fc2_input_quant: bool = True, pre_act_variant: bool = False,
            batched: bool = False) -> dict:
    """One MoE layer forward in fp64 (except the fp32 quantizer arithmetic).

    tokens: None for every token, or a list of token ids whose outputs are
    wanted (FC1 still runs over every route when the FC2 input has one
    per-tensor scale, because that scale is the amax over all routes).
    batched: FC1 and FC2 as one fp64 matrix product per expert over its routes
    (fc1_rows / fc2_rows) instead of one matrix-vector product per route; the
    results differ only in the fp64 summation order.
    fc2_input_quant=False and pre_act_variant=True are test-only switches
    (linearity check of the placement; the deliberately wrong pre-activation
    scaling) and are never used for parity.
    """
    assert mode in MODES
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    E = logits.shape[1]
    I = W.I
    out = {}
    ids, p = route(logits, K)                                        # S1
    counts, offsets, r2r, rt2row = permute(ids, E)                   # S2
    out.update(ids=ids, p=p, counts=counts, offsets=offsets, row_to_route=r2r,
               route_to_row=rt2row)
    xq = quantize_x(x_bits, mode, threads)                           # S3
    out["xq"] = xq

    toks = list(range(T)) if tokens is None else [int(t) for t in tokens]
    want = [t * K + k for t in toks for k in range(K)]
    per_tensor_fc2 = mode == "w4a4_tensor" and fc2_input_quant
    fc1_routes = list(range(T * K)) if per_tensor_fc2 else want
    W.ensure({int(ids.flat[r]) for r in fc1_routes}, threads)

    def activate(r, h):                                              # S5 (act, placement)
        a = np.empty(I, np.float64)
        lib().orc_activation(ACT_SWIGLU if act == "swiglu" else ACT_RELU2, I,
                             _p(np.ascontiguousarray(h)), int(on_input), float(p.flat[r]),
                             int(pre_act_variant), _p(a))
        return a

    if not fc1_routes:
        a = np.zeros((0, I))
    elif batched:                                                    # S4, per expert
        groups = _by_expert(fc1_routes, ids)

        def one(item):
            e, rs = item
            h = W.fc1_rows(e, np.stack([xq["deq"](r // K) for r in rs]))
            return rs, [activate(r, h[i]) for i, r in enumerate(rs)]
        pos = {r: i for i, r in enumerate(fc1_routes)}
        a = np.empty((len(fc1_routes), I), np.float64)
        with _blas_single_thread() if threads > 1 else _nullctx():
            for rs, rows in _pmap(one, sorted(groups.items()), threads):
                for r, row in zip(rs, rows):
                    a[pos[r]] = row
    else:
        def fc1(r):                                                  # S4, per route
            return activate(r, W.fc1(int(ids.flat[r]), xq["deq"](r // K)))
        a = np.stack(_pmap(fc1, fc1_routes, threads))
    a_idx = {r: i for i, r in enumerate(fc1_routes)}
    out["a_routes"] = np.array(fc1_routes, np.int64)
    out["a"] = a

    # S5: FC2-input precision (FP32 value, then the mode's quantizer or BF16 store)
    a32 = a.astype(np.float32)
    if not fc2_input_quant:
        a2 = a
    elif mode == "w4a16":
        a2 = bf16_bits_to_f32(f32_to_bf16_bits(a32)).reshape(a32.shape).astype(np.float64)
    elif mode == "mxfp8":
        c2, s2 = mxfp8_quantize(a32, threads)
        out["a2q"] = {"codes": c2, "scales": s2}
        a2 = mxfp8_dequant(c2, s2)
    else:
        per_row = mode in PER_ROW_MODES
        c2, s2, g2 = nvfp4_quantize(a32, per_row, threads, four_over_six=mode == "w4a4_token_4o6")
        out["a2q"] = {"codes": c2, "scales": s2, "g": g2}
        if mode == "w4a4_token_mxfp4":
            mc2, ms2 = mxfp4_reblock(c2, s2, threads)
            out["a2q"].update(mx_codes=mc2, mx_scales=ms2)
            a2 = mxfp4_dequant(mc2, ms2, g2, per_row)
        else:
            a2 = nvfp4_dequant(c2, s2, g2, per_row)

    # S6 + S7
    o, y = fc2_finalize(W, ids, p, K, on_input, toks, lambda r: a2[a_idx[r]], threads, batched)
    out["o"] = o
    out["tokens"] = np.array(toks, np.int64)
    out["y"] = y
    return out
