"""Shared helpers for the GPU parity tests: seeded inputs, the oracle run, blob
unpacking (host logic) and the comparison bars."""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import reference as R
from synth_inputs import make_expert_weights, make_logits, make_x
from synth_inputs.gen import STREAM_W1, STREAM_W2, make_weight

# Output bar: max|err| <= 2e-2 * rms(ref) and ||err||_F / ||ref||_F <= 1e-2,
# with the GPU's bf16 output compared against the unrounded fp64 oracle.
MAX_ERR_RMS = 2e-2
REL_FRO = 1e-2
TOPW_REL = 1e-6
# The output is bf16 by the interface: rounding the GPU's fp32 result y32 to
# bf16 (8 significant bits, round to nearest even) moves it by at most half a
# bf16 ulp of y32, and that half ulp is at most half an ulp of the rounded
# value y_gpu (RNE never lands in a lower binade). On heavy-tailed outputs that
# rounding alone can exceed 2e-2 * rms (measured up to 2.5e-2 on shapes outside
# the named workloads), so tests of arbitrary shapes bound the error beyond it.


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().float().numpy().astype(np.float64)


def half_ulp_bf16(y: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at each value: 2^(floor(log2|y|) - 8) (0 for y = 0)."""
    m, ex = np.frexp(np.abs(y))            # |y| = m 2^ex, m in [0.5, 1)
    return np.where(y != 0, np.ldexp(1.0, ex - 9), 0.0)


def out_errors(y_gpu: np.ndarray, y_ref: np.ndarray, round_allow=False):
    """max|err|/rms and the relative Frobenius error; with round_allow the max
    is taken over |err| - half_ulp_bf16(y_gpu) (the error beyond the output's
    own bf16 rounding)."""
    err = y_gpu - y_ref
    rms = math.sqrt(float(np.mean(y_ref * y_ref)))
    e = np.abs(err) - half_ulp_bf16(y_gpu) if round_allow else np.abs(err)
    max_rel = float(np.max(e)) / rms
    fro = float(np.linalg.norm(err) / np.linalg.norm(y_ref))
    return max_rel, fro


def assert_output_close(y_gpu: np.ndarray, y_ref: np.ndarray, what="", round_allow=False):
    max_rel, fro = out_errors(y_gpu, y_ref, round_allow)
    beyond = " beyond bf16 rounding" if round_allow else ""
    assert max_rel <= MAX_ERR_RMS and fro <= REL_FRO, \
        f"{what}: max|err|{beyond}/rms={max_rel:.3e} (bar {MAX_ERR_RMS}), rel Frobenius={fro:.3e} (bar {REL_FRO})"
    return max_rel, fro


class Inputs:
    """Seeded inputs of one workload shape, generated on `gen_device` and
    mirrored to the other side so that the oracle and the GPU read identical
    bytes."""

    def __init__(self, T, H, I, E, K, act, logits_kind, seed=0, gen_device="cpu",
                 make_weights=True):
        self.T, self.H, self.I, self.E, self.K, self.act = T, H, I, E, K, act
        self.N1 = 2 * I if act == "swiglu" else I
        self.seed = seed
        self.x = make_x(seed, T, H, device=gen_device).cuda()
        self.logits = make_logits(seed, T, E, logits_kind, device=gen_device).cuda()
        self.w1 = self.w2 = None
        if make_weights:
            if gen_device == "cpu":
                w1, w2 = make_expert_weights(seed, E, self.N1, H, I)
                self.w1, self.w2 = w1.cuda(), w2.cuda()
            else:
                self.w1 = torch.empty((E, self.N1, H), dtype=torch.float32, device="cuda")
                self.w2 = torch.empty((E, H, I), dtype=torch.float32, device="cuda")
                for e in range(E):
                    self.w1[e] = make_weight(seed, STREAM_W1, e, self.N1, H, device="cuda")
                    self.w2[e] = make_weight(seed, STREAM_W2, e, H, I, device="cuda")

    def x_bits(self):
        return bits16(self.x)

    def logits_np(self):
        return self.logits.cpu().numpy()

    def provider(self, e):
        return self.w1[e].cpu().numpy(), self.w2[e].cpu().numpy()

    def oracle_weights(self, fmt):
        """fmt: "nvfp4", "mxfp8" or "mxfp4" (R.weight_format(mode))."""
        return R.QuantWeights(fmt, self.E, self.H, self.I, self.act, self.provider)


# ---------------------------------------------------------------------------
# blob unpacking (layout documented in csrc/moe_internal.h)
# ---------------------------------------------------------------------------
HEADER_FIELDS = ["magic0", "magic1", "version", "wfmt", "E", "H", "I", "N1", "act", "pad0"]


def blob_header(blob: np.ndarray) -> dict:
    w = blob[:40].view(np.uint32)
    h = dict(zip(HEADER_FIELDS, [int(v) for v in w]))
    offs = blob[40:40 + 64].view(np.uint64)
    for k, v in zip(["off_g1", "off_g2", "off_amax", "off_w1", "off_s1", "off_w2", "off_s2",
                     "total"], offs):
        h[k] = int(v)
    return h


def _logical_rows(N, swiglu_I):
    p = np.arange(N)
    if not swiglu_I:
        return p
    st = p >> 4
    return (st & 1) * swiglu_I + (st >> 1) * 16 + (p & 15)


def tile_scales(scales_b: np.ndarray, NT: int, KT: int, unit: int) -> np.ndarray:
    """One expert's weight-scale bytes as stored (per group of four 16-row
    strips and K step, each lane's scale units of the four strips side by
    side; unit = 1 byte for MXFP8/MXFP4, 4 bytes for NVFP4) -> the same bytes
    in micro-tile order [NT][KT][tile scale bytes]."""
    S = 64 if unit == 1 else 128
    b = scales_b.reshape(NT // 4, KT, S // unit, 4, unit)   # group, step, unit, strip in group, byte
    return np.ascontiguousarray(b.transpose(0, 3, 1, 2, 4)).reshape(-1)


def unpack_nvfp4_matrix(codes_b: np.ndarray, scales_b: np.ndarray, N: int, K: int, swiglu_I=0):
    """Blob bytes of one expert's NVFP4 matrix -> (codes [N][K], scales [N][K/16])
    in logical (checkpoint) order."""
    NT, KT = N // 16, K // 128
    scales_b = tile_scales(scales_b, NT, KT, 4)
    t = codes_b.reshape(NT, KT, 64, 4, 4)           # tile, lane, dword j, byte
    lo, hi = t & 15, t >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(NT, KT, 64, 4, 8)  # element e = 2*byte + half
    lane = np.arange(64)
    out = np.empty((N, K), np.uint8)
    for j in range(4):
        for q in range(4):
            ls = lane[q * 16:(q + 1) * 16]
            # rows nt*16 + ls%16, k = kt*128 + 32 j + 8 q + e
            blk = nib[:, :, ls, j, :]                # NT, KT, 16, 8
            blk = blk.transpose(0, 2, 1, 3)          # NT, 16, KT, 8
            for e in range(8):
                out.reshape(NT, 16, KT, 128)[:, :, :, 32 * j + 8 * q + e] = blk[..., e]
    s = scales_b.reshape(NT, KT, 2, 16, 4)          # par, row, byte j
    sc = np.empty((N, K // 16), np.uint8)
    scv = sc.reshape(NT, 16, KT, 8)
    for par in range(2):
        for j in range(4):
            scv[:, :, :, 2 * j + par] = s[:, :, par, :, j].transpose(0, 2, 1)
    rows = _logical_rows(N, swiglu_I)
    outl = np.empty_like(out)
    scl = np.empty_like(sc)
    outl[rows] = out
    scl[rows] = sc
    return outl, scl


def unpack_mxfp8_matrix(codes_b: np.ndarray, scales_b: np.ndarray, N: int, K: int, swiglu_I=0):
    NT, KT = N // 16, K // 128
    scales_b = tile_scales(scales_b, NT, KT, 1)
    t = codes_b.reshape(NT, KT, 4, 16, 32)          # tile, q, row, byte
    out = np.empty((N, K), np.uint8)
    ov = out.reshape(NT, 16, KT, 128)
    for q in range(4):
        blk = t[:, :, q].transpose(0, 2, 1, 3)      # NT, 16, KT, 32
        ov[:, :, :, 16 * q:16 * q + 16] = blk[..., :16]
        ov[:, :, :, 64 + 16 * q:64 + 16 * q + 16] = blk[..., 16:]
    s = scales_b.reshape(NT, KT, 4, 16)             # block, row
    sc = np.empty((N, K // 32), np.uint8)
    scv = sc.reshape(NT, 16, KT, 4)
    for b in range(4):
        scv[:, :, :, b] = s[:, :, b, :].transpose(0, 2, 1)
    rows = _logical_rows(N, swiglu_I)
    outl = np.empty_like(out)
    scl = np.empty_like(sc)
    outl[rows] = out
    scl[rows] = sc
    return outl, scl


def unpack_mxfp4_matrix(codes_b: np.ndarray, scales_b: np.ndarray, N: int, K: int, swiglu_I=0):
    """MXFP4 micro-tiles: lane l = row (l % 16) + 16 q holds 16 bytes = the row's
    32-block q of the tile (even element in the low nibble); scale byte l."""
    NT, KT = N // 16, K // 128
    scales_b = tile_scales(scales_b, NT, KT, 1)
    t = codes_b.reshape(NT, KT, 4, 16, 16)          # tile, q, row, byte
    nib = np.stack([t & 15, t >> 4], axis=-1).reshape(NT, KT, 4, 16, 32)
    out = np.empty((N, K), np.uint8)
    ov = out.reshape(NT, 16, KT, 128)
    for q in range(4):
        ov[:, :, :, 32 * q:32 * q + 32] = nib[:, :, q].transpose(0, 2, 1, 3)
    s = scales_b.reshape(NT, KT, 4, 16)             # block, row
    sc = np.empty((N, K // 32), np.uint8)
    scv = sc.reshape(NT, 16, KT, 4)
    for b in range(4):
        scv[:, :, :, b] = s[:, :, b, :].transpose(0, 2, 1)
    rows = _logical_rows(N, swiglu_I)
    outl = np.empty_like(out)
    scl = np.empty_like(sc)
    outl[rows] = out
    scl[rows] = sc
    return outl, scl


def unpack_expert(blob: np.ndarray, e: int):
    """(W1 codes, W1 scales, g1, W2 codes, W2 scales, g2) of expert e."""
    h = blob_header(blob)
    E, H, I, N1 = h["E"], h["H"], h["I"], h["N1"]
    nv, mx4 = h["wfmt"] == 0, h["wfmt"] == 2
    tb, sb = (1024, 128) if nv else ((1024, 64) if mx4 else (2048, 64))
    t1 = (N1 // 16) * (H // 128)
    t2 = (H // 16) * (I // 128)
    sw = I if h["act"] == 0 else 0
    c1 = blob[h["off_w1"] + e * t1 * tb: h["off_w1"] + (e + 1) * t1 * tb]
    s1 = blob[h["off_s1"] + e * t1 * sb: h["off_s1"] + (e + 1) * t1 * sb]
    c2 = blob[h["off_w2"] + e * t2 * tb: h["off_w2"] + (e + 1) * t2 * tb]
    s2 = blob[h["off_s2"] + e * t2 * sb: h["off_s2"] + (e + 1) * t2 * sb]
    g1 = blob[h["off_g1"] + 4 * e: h["off_g1"] + 4 * e + 4].view(np.float32)[0]
    g2 = blob[h["off_g2"] + 4 * e: h["off_g2"] + 4 * e + 4].view(np.float32)[0]
    unpack = unpack_nvfp4_matrix if nv else (unpack_mxfp4_matrix if mx4 else unpack_mxfp8_matrix)
    w1c, w1s = unpack(c1, s1, N1, H, sw)
    w2c, w2s = unpack(c2, s2, H, I, 0)
    return w1c, w1s, g1, w2c, w2s, g2


def unpack_nibbles(packed: np.ndarray, n: int) -> np.ndarray:
    """[rows][n/2] packed E2M1 bytes (even element in the low nibble) -> [rows][n]."""
    p = packed.reshape(-1, n // 2)
    return np.stack([p & 15, p >> 4], axis=-1).reshape(-1, n)


# ---------------------------------------------------------------------------
# FC1 + activation (pre-quantization) parity and rounding-decision ambiguity
# ---------------------------------------------------------------------------
# Bound on |a_gpu - a_oracle| / max_i |a_oracle[r, i]| for one route's FC2
# input before quantization. The f16/bf16 matrix-core paths accumulate in fp32
# (measured <= 2.5e-7 at H=256); the block-scaled fp8 matrix core rounds
# inside each 128-deep instruction more coarsely (measured up to 7.4e-5), so
# its bound is wider. Both bounds carry a margin over the measurements.
TAU = {"w4a4_tensor": 2.0 ** -18, "w4a4_token": 2.0 ** -18, "w4a4_token_4o6": 2.0 ** -18,
       "w4a4_token_mxfp4": 2.0 ** -11, "w4a16": 2.0 ** -18,
       "mxfp8": 2.0 ** -11}


def check_prequant(a_gpu_perm: np.ndarray, ref: dict, mode: str, what=""):
    """a_gpu_perm: the GPU's FC2 input before quantization, [R][I] in permuted
    row order (fp32, or bf16 values for W4A16). Compares the oracle's routes:
    |a_gpu - a_ref| <= TAU * rowmax (+ half a bf16 ulp of the stored value for
    W4A16, whose FC2 input is that rounding of the fp32 activation)."""
    routes = ref["a_routes"]
    rows = ref["route_to_row"][routes]
    a_ref = ref["a"]
    a_g = a_gpu_perm[rows].astype(np.float64)
    scale = np.abs(a_ref).max(1, keepdims=True) + 1e-300
    bound = TAU[mode] * scale
    if mode == "w4a16":
        bound = bound + half_ulp_bf16(a_g)
    excess = np.abs(a_g - a_ref) - bound
    assert np.all(excess <= 0), \
        f"{what}: FC1+activation differs from the oracle beyond the bound " \
        f"(worst |diff|/rowmax = {float((np.abs(a_g - a_ref) / scale).max()):.3e})"


def check_a2_mxfp8(codes_perm: np.ndarray, scales_perm: np.ndarray, ref: dict, what=""):
    """MXFP8 FC2 input quantized in the FC1 epilogue (no pre-quantization copy
    exists). codes_perm [R][I] E4M3, scales_perm [R][I/32] E8M0, permuted row
    order. Against the oracle's FP32 value v of each element, with
    eps = TAU * rowmax (the FC1 accumulation-order allowance):
      - the block exponent is one the block max can take within +-eps:
        floor(log2(amax)) - 8 for amax in [amax_ref - eps, amax_ref + eps];
      - the decoded element lies within eps plus half an E4M3 step (at its
        own magnitude and the block scale) of v, or is the saturated +-448
        times the block scale where |v| + eps reaches the saturation range."""
    routes = ref["a_routes"]
    rows = ref["route_to_row"][routes]
    a32 = ref["a"].astype(np.float32).astype(np.float64)
    n, I = a32.shape
    c = codes_perm[rows]
    sc = scales_perm[rows]
    deq = R.mxfp8_dequant(c, sc)
    X = sc.astype(np.int64) - 127
    eps = TAU["mxfp8"] * np.abs(ref["a"]).max(1, keepdims=True)
    blk = np.abs(a32).reshape(n, I // 32, 32).max(2)
    e_blk = eps.repeat(I // 32, 1)

    def expo(a):
        out = np.full(a.shape, -127, np.int64)
        nz = a > 0
        out[nz] = np.clip(np.floor(np.log2(a[nz])).astype(np.int64) - 8, -127, 127)
        return out

    lo, hi = expo(np.maximum(blk - e_blk, 0.0)), expo(blk + e_blk)
    assert np.all((X >= lo) & (X <= hi)), f"{what}: MXFP8 block exponent outside the allowed range"
    Xe = np.repeat(X, 32, axis=1).astype(np.float64)
    g = np.abs(deq) * np.exp2(-Xe)
    step = np.where(g >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(g, 2.0 ** -6))) - 3), 2.0 ** -9)
    bound = eps + 0.5 * step * np.exp2(Xe)
    err = np.abs(deq - a32)
    sat = (np.abs(deq) == 448.0 * np.exp2(Xe)) & (np.abs(a32) + eps >= 448.0 * np.exp2(Xe))
    bad = (err > bound) & ~sat
    assert not bad.any(), \
        f"{what}: {int(bad.sum())} MXFP8 FC2-input elements off the oracle's rounding cell"




# ---------------------------------------------------------------------------
# the FC2 input the GPU produced (S5) and the layer output
# ---------------------------------------------------------------------------
# E2M1 rounding cells: code magnitude m is the round-to-nearest-even result
# for |u| in [CELL_LO[m], CELL_HI[m]] (ties belong to the even neighbour; the
# checks below accept either side of a tie anyway).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
CELL_LO = np.array([0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
CELL_HI = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, np.inf])
_E4M3_TABLE = None


def _e4m3_table():
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = np.array([R.e4m3_decode(c) if (c & 0x7F) != 0x7F else np.nan
                                for c in range(256)])
    return _E4M3_TABLE


def _fl32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


class Fc2Input:
    """The FC2 input of one forward as the GPU left it in the workspace, rows in
    permuted order: `pre` is the value before quantization (fp32 for W4A4,
    the stored bf16 values for W4A16, None for MXFP8, which quantizes in the
    FC1 epilogue), `codes` unpacked one per byte, `scales`, and `g` ([1] per
    tensor or [R] per route, NVFP4 only)."""

    def __init__(self, mode, pre=None, codes=None, scales=None, g=None, mx_codes=None,
                 mx_scales=None):
        self.mode, self.pre, self.codes, self.scales, self.g = mode, pre, codes, scales, g
        self.mx_codes, self.mx_scales = mx_codes, mx_scales   # MXFP4 re-blocked (mode 5)

    def dequant_row(self, row: int) -> np.ndarray:
        """The fp64 FC2 input row the GPU's FC2 consumed (its own codes)."""
        m = self.mode
        if m == "w4a16":
            return self.pre[row].astype(np.float64)
        if m == "mxfp8":
            return R.mxfp8_dequant(self.codes[row:row + 1], self.scales[row:row + 1])[0]
        if m == "w4a4_token_mxfp4":
            return R.mxfp4_dequant(self.mx_codes[row:row + 1], self.mx_scales[row:row + 1],
                                   self.g[row:row + 1])[0]
        per_row = m in R.PER_ROW_MODES
        g = self.g[row:row + 1] if per_row else self.g[:1]
        return R.nvfp4_dequant(self.codes[row:row + 1], self.scales[row:row + 1], g,
                               per_row=per_row)[0]


def read_fc2_input(moe, d, ws, T: int, K: int, mode: str) -> Fc2Input:
    R_, I = T * K, d.I

    def v(name):
        return moe.workspace_view(d, ws, T, K, mode, name).cpu().numpy()
    if mode == "w4a16":
        return Fc2Input(mode, pre=moe.workspace_view(d, ws, T, K, mode, "a2_pre").float()
                        .cpu().numpy().reshape(R_, I))
    if mode == "mxfp8":
        return Fc2Input(mode, codes=v("a2_codes").reshape(R_, I),
                        scales=v("a2_scales").reshape(R_, I // 32))
    gi = Fc2Input(mode, pre=v("a2_pre").reshape(R_, I),
                  codes=unpack_nibbles(v("a2_codes"), I).reshape(R_, I),
                  scales=v("a2_scales").reshape(R_, I // 16),
                  g=v("a2_g")[:R_ if mode in R.PER_ROW_MODES else 1])
    if mode == "w4a4_token_mxfp4":
        gi.mx_codes = unpack_nibbles(v("a2_mx_codes"), I).reshape(R_, I)
        gi.mx_scales = v("a2_mx_scales").reshape(R_, I // 32)
    return gi


def check_s5_quantizer(gi: Fc2Input, threads: int = 1, what=""):
    """NVFP4 FC2-input quantization, bit-exact: the GPU's codes, block scales
    and global scale(s) of every route equal the oracle's quantizer applied to
    the GPU's own fp32 values before quantization (per-tensor g from the amax
    of all R*I values, or one g per route)."""
    per_row = gi.mode in R.PER_ROW_MODES
    codes, sf, g = R.nvfp4_quantize(gi.pre, per_row, threads,
                                    four_over_six=gi.mode == "w4a4_token_4o6")
    assert np.array_equal(gi.g, g), f"{what}: FC2-input global scale(s) differ from the oracle's quantizer"
    assert np.array_equal(gi.scales, sf), \
        f"{what}: {int((gi.scales != sf).sum())} FC2-input block scales differ from the oracle's quantizer"
    assert np.array_equal(gi.codes, codes), \
        f"{what}: {int((gi.codes != codes).sum())} FC2-input codes differ from the oracle's quantizer"
    if gi.mode == "w4a4_token_mxfp4":  # the re-blocking of the GPU's own NVFP4, bit-exact
        mc, ms = R.mxfp4_reblock(gi.codes, gi.scales, threads)
        assert np.array_equal(gi.mx_scales, ms), f"{what}: re-blocked E8M0 scales differ"
        assert np.array_equal(gi.mx_codes, mc), \
            f"{what}: {int((gi.mx_codes != mc).sum())} re-blocked MXFP4 codes differ"


def check_a2_nvfp4(gi: Fc2Input, ref: dict, what=""):
    """NVFP4 FC2 input against the oracle's fp64 activation v of each sampled
    route (twin of check_a2_mxfp8), with eps = TAU * rowmax the FC1
    accumulation-order allowance (the GPU's fp32 values may differ from v by
    up to eps):
      - the global scale is fl32(fl32(A)/2688) for an amax A within eps of
        the oracle's (over all routes per tensor, over the row per route);
      - each block scale is the E4M3 rounding of fl32(a_b / fl32(6 g)) for a
        block max a_b within eps of the oracle's, g being the GPU's own (for
        the 4-over-6 contract: global scale fl32(A)/1536, and the block
        scale either that or the max-to-4 one, fl32(a_b / fl32(4 g)));
      - each code's E2M1 rounding cell, at the decode scale d = fl32(sf g) of
        the GPU's own scales, lies within eps / d of v / d, with v's sign
        wherever |v| > eps; a zero decode scale leaves sign-only codes."""
    mode = gi.mode
    routes = ref["a_routes"]
    rows = ref["route_to_row"][routes]
    v = ref["a"]
    n, I = v.shape
    tau = TAU[mode]
    rowmax = np.abs(v).max(1)
    eps = tau * rowmax
    tab = _e4m3_table()
    # global scale
    f46 = mode == "w4a4_token_4o6"
    gdiv = 1536.0 if f46 else 2688.0
    if mode in R.PER_ROW_MODES:
        g = gi.g[rows].astype(np.float64)
        glo = _fl32(_fl32(np.maximum(rowmax - eps, 0.0)) / gdiv)
        ghi = _fl32(_fl32(rowmax + eps) / gdiv)
    else:
        assert len(routes) == ref["route_to_row"].size, "per-tensor scale needs every route"
        A = float(rowmax.max())
        g = np.full(n, float(gi.g[0]))
        glo = np.full(n, float(_fl32(_fl32(max(A - tau * A, 0.0)) / 2688.0)))
        ghi = np.full(n, float(_fl32(_fl32(A + tau * A) / 2688.0)))
    bad_g = (g < glo) | (g > ghi)
    assert not bad_g.any(), f"{what}: {int(bad_g.sum())} FC2-input global scales outside the allowed range"
    # block scales
    ab = np.abs(v).reshape(n, I // 16, 16).max(2)
    sf = gi.scales[rows].astype(np.int64)
    enc = np.vectorize(lambda x: R.e4m3_encode(float(x)), otypes=[np.int64])

    def scale_range(top):
        top_g = _fl32(top * g)[:, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            s_lo = np.where(top_g > 0, _fl32(_fl32(np.maximum(ab - eps[:, None], 0.0)) / top_g), 0.0)
            s_hi = np.where(top_g > 0, _fl32(_fl32(ab + eps[:, None]) / top_g), 0.0)
        return enc(s_lo), enc(s_hi), top_g
    lo, hi, six_g = scale_range(6.0)
    ok_s = (sf >= lo) & (sf <= hi)
    if f46:
        lo4, hi4, _ = scale_range(4.0)
        ok_s |= (sf >= lo4) & (sf <= hi4)
    bad_s = ~ok_s | ((six_g == 0) & (sf != 0))
    assert not bad_s.any(), f"{what}: {int(bad_s.sum())} FC2-input block scales outside the allowed range"
    # element codes
    c = gi.codes[rows].astype(np.int64)
    m, neg = c & 7, (c & 8) != 0
    d = _fl32(tab[sf] * g[:, None])                     # [n, I/16]
    d = np.repeat(d, 16, axis=1)
    e = np.repeat(eps[:, None], I, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(d > 0, np.abs(v) / d, 0.0)
        du = np.where(d > 0, e / d, 0.0)
    in_cell = (u >= CELL_LO[m] - du) & (u <= CELL_HI[m] + du)
    ok = np.where(d > 0, in_cell, m == 0)
    sign_ok = (neg == np.signbit(v)) | (np.abs(v) <= e)
    bad = ~(ok & sign_ok)
    assert not bad.any(), \
        f"{what}: {int(bad.sum())} NVFP4 FC2-input codes off the oracle's rounding cell " \
        f"(first at sampled route {int(np.argwhere(bad)[0][0])})"


def check_fc2_input(gi: Fc2Input, ref: dict, threads: int = 1, what=""):
    """Every check of the FC2 input the GPU produced (S5)."""
    if gi.mode == "mxfp8":
        return check_a2_mxfp8(gi.codes, gi.scales, ref, what)
    check_prequant(gi.pre, ref, gi.mode, what)
    if gi.mode != "w4a16":
        check_s5_quantizer(gi, threads, what)
        check_a2_nvfp4(gi, ref, what)


def expected_from_own_fc2_input(gi: Fc2Input, ref: dict, W, K: int, on_input: bool,
                                threads: int = 1) -> np.ndarray:
    """The oracle's FC2 and finalize (fp64) run on the FC2 input the GPU itself
    produced, for the oracle's tokens: the layer output the GPU must reproduce
    given its own FC2-input rounding decisions, which check_fc2_input has
    already tied to the oracle's FC1 and activation."""
    r2row = ref["route_to_row"]
    _, y = R.fc2_finalize(W, ref["ids"], ref["p"], K, on_input, ref["tokens"],
                          lambda r: gi.dequant_row(int(r2row[r])), threads, batched=True)
    return y


def check_layer_output(y_gpu: np.ndarray, gi: Fc2Input, ref: dict, W, K: int, on_input: bool,
                       what="", round_allow=False, threads: int = 1):
    """The layer output y_gpu (bf16 values, rows of ref["tokens"]) at the plain
    bar (max|err| <= 2e-2 rms, relative Frobenius <= 1e-2; with round_allow
    the max counts the error beyond the output's own bf16 rounding) against
    the oracle's FC2 and finalize on the GPU's own FC2 input, after the FC2
    input itself is checked against the oracle. Nothing is re-taken. The
    plain comparison with the oracle's own end-to-end result is returned
    beside it (it differs only through FC2-input rounding decisions within
    the FC1 accumulation allowance)."""
    check_fc2_input(gi, ref, threads, what)
    y_exp = expected_from_own_fc2_input(gi, ref, W, K, on_input, threads)
    own = assert_output_close(y_gpu, y_exp, f"{what} (vs oracle FC2+finalize on the GPU's FC2 input)",
                              round_allow)
    plain = out_errors(y_gpu, ref["y"], round_allow)
    print(f"{what}: vs own-FC2-input oracle max|err|/rms={own[0]:.3e} fro={own[1]:.3e}; "
          f"vs end-to-end oracle max|err|/rms={plain[0]:.3e} fro={plain[1]:.3e}", flush=True)
    return {"own": own, "plain": plain, "own_plain": out_errors(y_gpu, y_exp, False),
            "plain_nr": out_errors(y_gpu, ref["y"], False)}


def check_layer(moe, d, ws, y, ref, W, T: int, K: int, mode: str, on_input: bool, what="",
                round_allow=False, threads: int = 8):
    """check_layer_output on a forward's workspace and bf16 output tensor."""
    gi = read_fc2_input(moe, d, ws, T, K, mode)
    yg = bf16_to_f64(y)[ref["tokens"]]
    return check_layer_output(yg, gi, ref, W, K, on_input, what, round_allow, threads)
