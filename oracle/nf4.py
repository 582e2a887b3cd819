"""Plain NumPy oracle of blockwise NF4 quantization and the 4-bit-storage /
16-bit-compute linear layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here is tuned:
each step is written the way the pages state it, with NumPy's IEEE binary32
operations (round-to-nearest-even, no fusion) wherever the stored format is
binary32, and binary64 for the reference matmul.

Sources (five web pages about bitsandbytes; cited by page and section):

* mlqm.cn bitsandbytes article (news/394670), section 3.2 "4bit: NF4":
  16 non-uniform levels placed by the normal density, dense near zero,
  sparse at the ends.
* same article, section 3.3 "double quantization": one scale per block,
  stored as FP32; the scales are themselves quantized a second time, saving a
  few tenths of a bit per parameter.
* same article, section 3.4 "compute dtype": weights are stored in 4 bits
  and dequantized to FP16/BF16 before the matrix multiply ("4-bit storage,
  16-bit compute").
* pomoai.com bitsandbytes overview, module list: ``bitsandbytes.functional``
  holds the blockwise quantization and the NF4 format; ``Linear4bit``
  replaces ``torch.nn.Linear`` (weight laid out [out_features, in_features]).

* same article, section 4 (the 4-bit loading options): the 4-bit quant type
  is ``nf4`` (the NormalFloat levels) or ``fp4`` (a plain 4-bit float,
  usually worse than nf4), and the compute dtype is BF16 or FP16; the
  csdn.net feature page (example 2) loads a model with FP4 the same way.

Parameters the pages leave open (blocksize 64, second-level groups of 256,
int8 second level with the mean removed, lower-index tie rule, the FP4 bit
layout) are the ones this path fixes; every such reading is noted where it
is used.
"""

from __future__ import annotations

import math
import statistics

import numpy as np

BLOCKSIZE = 64      # weights per first-level block (reading: fixed at 64)
DQ_GROUP = 256      # first-level scales per second-level group (reading)
ZERO_CODE = 7       # index of the exact 0.0 level in the ascending codebook
QUANT_TYPES = ("nf4", "fp4")
DTYPES = ("bf16", "f16")


# --------------------------------------------------------------------------
# bfloat16 <-> binary32
# --------------------------------------------------------------------------
def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to binary32.  Exact: bfloat16 is
    the top half of a binary32."""
    u = np.ascontiguousarray(bits, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(values) -> np.ndarray:
    """Round binary32 to bfloat16 with round-to-nearest, ties to even, and
    return the bit patterns (uint16).  The mlqm.cn article, section 3.4, has
    the weights dequantized to BF16 for the multiply; RNE is the IEEE default
    rounding (reading: the pages name no rounding mode)."""
    f = np.ascontiguousarray(values, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    # Add just under half an ulp of the kept part, plus one if the kept part
    # is odd: a tie then rounds to the even neighbour.
    kept_lsb = (u >> np.uint64(16)) & np.uint64(1)
    out = ((u + np.uint64(0x7FFF) + kept_lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():  # keep NaNs NaN (quiet bit set) instead of rounding to inf
        out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return out


def f16_bits_to_f32(bits) -> np.ndarray:
    """Widen IEEE binary16 bit patterns (uint16) to binary32 (exact)."""
    u = np.ascontiguousarray(bits, dtype=np.uint16)
    return u.view(np.float16).astype(np.float32)


def f32_to_f16_bits(values) -> np.ndarray:
    """Round binary32 to IEEE binary16 (round to nearest even, subnormals
    kept, overflow to infinity) and return the bit patterns.  FP16 is the
    other compute dtype of section 4 of the mlqm.cn article.  Library
    primitive: NumPy's float32 -> float16 conversion."""
    f = np.ascontiguousarray(values, dtype=np.float32)
    with np.errstate(over="ignore"):
        return f.astype(np.float16).view(np.uint16)


def bits_to_f32(bits, dtype: str = "bf16") -> np.ndarray:
    """16-bit patterns of the compute dtype ("bf16" or "f16") to binary32."""
    if dtype == "bf16":
        return bf16_bits_to_f32(bits)
    if dtype == "f16":
        return f16_bits_to_f32(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def f32_to_bits(values, dtype: str = "bf16") -> np.ndarray:
    """Round binary32 to the compute dtype ("bf16" or "f16"), RNE."""
    if dtype == "bf16":
        return f32_to_bf16_bits(values)
    if dtype == "f16":
        return f32_to_f16_bits(values)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# Step 1: the NF4 codebook
# --------------------------------------------------------------------------
# Probability offset of the outermost quantile.  Reading: the pages only say
# the levels follow the normal density with an exact zero; the construction
# below is the one of the QLoRA work the pages credit NF4 to (pomoai.com
# overview, QLoRA paragraph; mlqm.cn article section 5.4): the ends sit at
# the average of the 1/30 and 1/32 tail probabilities.
NF4_OFFSET = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)


def normal_quantile(p: float) -> float:
    """Inverse of the standard normal CDF, in binary64.

    Library primitive: Python's ``statistics.NormalDist.inv_cdf`` (Wichura's
    AS241 algorithm, relative error about 1e-16)."""
    return statistics.NormalDist(0.0, 1.0).inv_cdf(p)


def codebook() -> np.ndarray:
    """The 16 NF4 levels, ascending, as binary32.

    mlqm.cn article, section 3.2: the 16 levels are not evenly spaced but
    follow the normal density, dense near 0 and sparse at the two ends.
    Construction (reading, see NF4_OFFSET): 8 positive levels at the
    standard-normal quantiles of 8 probabilities evenly spaced from the offset
    down towards 1/2 (1/2 itself excluded), 7 negative levels mirrored from 7
    evenly spaced probabilities over the same span, and an exact 0.  All are
    divided by the outermost quantile so the ends are exactly -1 and +1.
    Arithmetic in binary64, one rounding to binary32 at the end.
    """
    top = normal_quantile(NF4_OFFSET)
    positive = [normal_quantile(NF4_OFFSET + i * (0.5 - NF4_OFFSET) / 8.0)
                for i in range(8)]
    negative = [-normal_quantile(NF4_OFFSET + i * (0.5 - NF4_OFFSET) / 7.0)
                for i in range(7)]
    values = sorted(negative + [0.0] + positive)
    return np.array([v / top for v in values], dtype=np.float64).astype(np.float32)


def thresholds(levels: np.ndarray) -> np.ndarray:
    """Decision thresholds T[0..len-2] for nearest-level encoding over
    ascending levels (15 for NF4).

    The midpoint m_i of levels i and i+1 is exact in binary64.  T_i is the
    smallest binary32 strictly above m_i, so that ``#{i : x >= T_i}`` is the
    index of the nearest level and a value exactly on a midpoint goes to the
    LOWER index (the tie rule this path fixes; the pages state none)."""
    L = np.asarray(levels, dtype=np.float32).astype(np.float64)
    out = np.empty(L.size - 1, dtype=np.float32)
    for i in range(L.size - 1):
        mid = (L[i] + L[i + 1]) / 2.0
        t = np.float32(mid)
        if float(t) <= mid:
            t = np.nextafter(t, np.float32(np.inf), dtype=np.float32)
        out[i] = t
    return out


# --------------------------------------------------------------------------
# Step 1b: the FP4 codebook (the other 4-bit quant type)
# --------------------------------------------------------------------------
def fp4_codebook() -> np.ndarray:
    """The 16 FP4 levels indexed by code, as binary32.

    mlqm.cn article, section 4: besides nf4 the 4-bit quant type may be
    ``fp4``, a plain 4-bit floating-point format; the pages give no bit
    layout.  Reading: the common E2M1 layout -- bit 3 the sign, bits 2-1 a
    biased exponent e, bit 0 a mantissa bit m; the magnitude is m/2 for
    e = 0 (zero and the one subnormal) and 2^(e-1) * (1 + m/2) otherwise,
    so codes 0..7 hold 0, 1/2, 1, 3/2, 2, 3, 4, 6.  Every level is divided
    by the largest magnitude, 6, so that the block absmax maps to +-1 as
    with NF4.  Binary64 arithmetic, one rounding to binary32."""
    out = []
    for c in range(16):
        sign = -1.0 if c & 8 else 1.0
        e = (c >> 1) & 3
        m = c & 1
        mag = m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
        out.append(sign * mag / 6.0)
    return np.array(out, dtype=np.float64).astype(np.float32)


def levels_by_code(quant_type: str = "nf4") -> np.ndarray:
    """Level of each 4-bit code (float32[16]): the ascending NF4 codebook, or
    the FP4 levels in code order."""
    if quant_type == "nf4":
        return codebook()
    if quant_type == "fp4":
        return fp4_codebook()
    raise ValueError(f"unknown quant type {quant_type!r}")


def sorted_codes(quant_type: str = "nf4") -> np.ndarray:
    """Codes of the distinct levels, by ascending level value.  NF4 codes
    are already in value order.  For FP4 both zero codes decode to 0; the
    encoder emits only code 0 (+0), so code 8 (-0) is left out and the 15
    remaining levels are sorted (reading)."""
    if quant_type == "nf4":
        return np.arange(16, dtype=np.uint8)
    levels = levels_by_code(quant_type)
    codes = [c for c in range(16) if c != 8]
    codes.sort(key=lambda c: float(levels[c]))
    return np.array(codes, dtype=np.uint8)


# --------------------------------------------------------------------------
# Steps 2-4: block absmax, normalise, encode, pack
# --------------------------------------------------------------------------
def _blocks(n: int, blocksize: int) -> int:
    return -(-n // blocksize)


def block_absmax(wf: np.ndarray, blocksize: int = BLOCKSIZE) -> np.ndarray:
    """a_b = max |w| over each run of ``blocksize`` consecutive elements of the
    flat weight (the last block may be short).  mlqm.cn article, section 3.3:
    one scale per block, stored as FP32; the absmax scale is the basic
    data-free quantizer the article points back to (section 2.3)."""
    wf = np.ascontiguousarray(wf, dtype=np.float32).ravel()
    n = wf.size
    nb = _blocks(n, blocksize)
    padded = np.zeros(nb * blocksize, dtype=np.float32)
    padded[:n] = np.abs(wf)
    return padded.reshape(nb, blocksize).max(axis=1)


def encode(wf: np.ndarray, absmax: np.ndarray, thr: np.ndarray,
           blocksize: int = BLOCKSIZE, order: np.ndarray | None = None,
           zero_code: int = ZERO_CODE) -> np.ndarray:
    """4-bit code of every weight (uint8 values 0..15).

    Normalise into [-1, 1] with the block's binary32 reciprocal,
    x = fl32(w * fl32(1 / a_b)) (reading: multiply by the reciprocal rather
    than divide), then count the thresholds at or below x, which picks the
    nearest level (section 3.2).  ``order`` maps that ascending level index
    to its code (identity for NF4, ``sorted_codes("fp4")`` for FP4).  A
    block whose absmax is 0 is all zero weights and takes the zero level's
    code for every element (reading).

    A block whose absmax is below 2^-100 is first scaled, weights and absmax
    alike, by 2^64 (exact for binary32 values that small): without it the
    reciprocal of an absmax at or below 2^-128 overflows to infinity, the
    zeros of the block turn into NaN and nothing is the nearest level any
    more.  For every absmax above 2^-128 the scaled form gives the same x as
    the plain one (the two products are the same real number), so only the
    blocks that used to overflow change."""
    wf = np.ascontiguousarray(wf, dtype=np.float32).ravel()
    n = wf.size
    block = np.arange(n) // blocksize
    a32 = absmax.astype(np.float32)
    tiny = a32 < np.float32(2.0 ** -100)
    pre = np.where(tiny, np.float32(2.0 ** 64), np.float32(1.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        recip = (np.float32(1.0) / (a32 * pre).astype(np.float32)).astype(np.float32)
        x = ((wf * pre[block]).astype(np.float32) * recip[block]).astype(np.float32)
    codes = np.zeros(n, dtype=np.uint8)
    with np.errstate(invalid="ignore"):
        for t in np.asarray(thr, dtype=np.float32):
            codes += (x >= t).astype(np.uint8)
    if order is not None:
        codes = np.asarray(order, dtype=np.uint8)[codes]
    zero_block = absmax[block] == 0
    codes[zero_block] = zero_code
    return codes


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte ("4-bit storage", section 3.4).  Reading: the even
    (first) element goes in the high nibble.  The element count must be
    even."""
    c = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    if c.size % 2:
        raise ValueError("odd element count cannot be packed two per byte")
    return ((c[0::2] << np.uint8(4)) | c[1::2]).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles."""
    p = np.ascontiguousarray(packed, dtype=np.uint8).ravel()
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> np.uint8(4)
    out[1::2] = p & np.uint8(0x0F)
    return out


# --------------------------------------------------------------------------
# Step 5: double quantization of the first-level scales
# --------------------------------------------------------------------------
def double_quant(absmax: np.ndarray, group: int = DQ_GROUP):
    """Quantize the FP32 block scales a second time (section 3.3: first
    quantization gives the scales, the second compresses them).

    Readings: remove the mean of all scales, then symmetric absmax int8
    quantization in groups of ``group`` consecutive scales (last group may be
    short).

    * mean: S = sum of a_b, correctly rounded to binary64 (``math.fsum``),
      mu = fl32(S / nb) with the division in binary64;
    * c_b = fl32(a_b - mu);
    * s_g = max |c_b| over the group;
    * q_b = round-half-even(fl32(fl32(c_b / s_g) * 127)) in [-127, 127];
      a group with s_g = 0 stores q_b = 0.

    Returns (q int8[nb], s float32[ng], mu float32).
    """
    a = np.ascontiguousarray(absmax, dtype=np.float32).ravel()
    nb = a.size
    total = math.fsum(a.astype(np.float64).tolist())
    mean = np.float32(total / nb)
    centred = (a - mean).astype(np.float32)
    ng = _blocks(nb, group)
    padded = np.zeros(ng * group, dtype=np.float32)
    padded[:nb] = np.abs(centred)
    s = padded.reshape(ng, group).max(axis=1).astype(np.float32)
    g = np.arange(nb) // group
    q = np.zeros(nb, dtype=np.int8)
    live = s[g] > 0
    t = (centred[live] / s[g][live]).astype(np.float32)
    u = (t * np.float32(127.0)).astype(np.float32)
    q[live] = np.rint(u).astype(np.int8)
    return q, s, mean


# --------------------------------------------------------------------------
# Step 5b: the "dynamic" 8-bit map for the second level
# --------------------------------------------------------------------------
DQ_MAPS = ("linear", "dynamic")


def dynamic_map() -> np.ndarray:
    """The 256 values of the "dynamic" 8-bit quantization map, ascending, as
    binary32.

    The csdn.net feature page (section 1, item 5) lists quantile, linear and
    dynamic 8-bit quantization among the library's types, and the mlqm.cn
    article (section 3.3) quantizes the FP32 block scales a second time; no
    page defines the dynamic map.  Reading: dynamic tree quantization as
    published by Dettmers (8-bit approximations for parallelism in deep
    learning, 2016; reused as the 8-bit code of block-wise quantization,
    2021).  After the sign bit, E zero bits give a decimal exponent 10^-E, a
    one bit ends them, and the remaining 6 - E bits index 2^(6-E) equal bins
    of [0.1, 1], the value being the bin's midpoint:
    |v| = 10^-E * (0.1 + 0.9 (f + 1/2) / 2^(6-E)), E = 0..6.  That gives 127
    magnitudes of each sign; 0 and 1.0 complete the 256.  Binary64
    arithmetic, one rounding to binary32, sorted."""
    vals = [0.0, 1.0]
    for e in range(7):
        nf = 2 ** (6 - e)
        for f in range(nf):
            mag = 10.0 ** (-e) * (0.1 + 0.9 * (f + 0.5) / nf)
            vals += [mag, -mag]
    return np.array(sorted(vals), dtype=np.float64).astype(np.float32)


def double_quant_dynamic(absmax: np.ndarray, group: int = DQ_GROUP):
    """Second-level quantization with the dynamic map (reading, see
    dynamic_map): the mean and the group scales as in ``double_quant``;
    t_b = fl32(c_b / s_g) (correctly rounded division), and the code q_b is
    the index of the map value nearest t_b, exact ties to the lower index
    (the rule of the 4-bit codes: thresholds just above the midpoints).  A
    group with s_g = 0 stores the index of 0.0.

    Returns (q uint8[nb], s float32[ng], mu float32)."""
    a = np.ascontiguousarray(absmax, dtype=np.float32).ravel()
    nb = a.size
    total = math.fsum(a.astype(np.float64).tolist())
    mean = np.float32(total / nb)
    centred = (a - mean).astype(np.float32)
    ng = _blocks(nb, group)
    padded = np.zeros(ng * group, dtype=np.float32)
    padded[:nb] = np.abs(centred)
    s = padded.reshape(ng, group).max(axis=1).astype(np.float32)
    g = np.arange(nb) // group
    dmap = dynamic_map()
    thr = thresholds(dmap)
    zero_index = int(np.flatnonzero(dmap == 0)[0])
    q = np.full(nb, zero_index, dtype=np.uint8)
    live = s[g] > 0
    t = (centred[live] / s[g][live]).astype(np.float32)
    q[live] = np.searchsorted(thr, t, side="right").astype(np.uint8)
    return q, s, mean


def block_scales(state: dict) -> np.ndarray:
    """The per-block scale the dequantizer uses, binary32.

    Without double quant it is the stored a_b.  With the linear int8 second
    level (reading): step_g = fl32(s_g / 127), a_hat_b =
    fl32(fl32(q_b * step_g) + mu); with the dynamic map: a_hat_b =
    fl32(fl32(map[q_b] * s_g) + mu).  Each operation is rounded on its own
    (no fused multiply-add)."""
    if not state["double_quant"]:
        return np.asarray(state["absmax"], dtype=np.float32)
    s = np.asarray(state["absmax2"], dtype=np.float32)
    mean = np.float32(state["absmax_mean"])
    group = state.get("group", DQ_GROUP)
    if state.get("dq_map", "linear") == "dynamic":
        q = np.asarray(state["absmax"], dtype=np.uint8)
        g = np.arange(q.size) // group
        prod = (dynamic_map()[q] * s[g]).astype(np.float32)
        return (prod + mean).astype(np.float32)
    q = np.asarray(state["absmax"], dtype=np.int8)
    step = (s / np.float32(127.0)).astype(np.float32)
    g = np.arange(q.size) // group
    prod = (q.astype(np.float32) * step[g]).astype(np.float32)
    return (prod + mean).astype(np.float32)


def quantize(w_bits: np.ndarray, double_quant_on: bool,
             blocksize: int = BLOCKSIZE, group: int = DQ_GROUP,
             quant_type: str = "nf4", dq_map: str = "linear") -> dict:
    """Blockwise 4-bit (NF4 or FP4) quantize-on-load of a bfloat16 weight
    (bit patterns).

    Returns a dict with ``codes`` (uint8[n]), ``packed`` (uint8[n/2]) and the
    quant state: ``absmax`` (float32[nb], or int8[nb] with double quant),
    ``absmax2`` (float32[ng]) and ``absmax_mean`` (float32) with double
    quant, plus ``absmax_fp32`` (the first-level scales before the second
    quantization)."""
    wf = bf16_bits_to_f32(np.ascontiguousarray(w_bits).ravel())
    levels = levels_by_code(quant_type)
    order = sorted_codes(quant_type)
    thr = thresholds(levels[order])
    zero_code = int(order[int(np.flatnonzero(levels[order] == 0)[0])])
    a = block_absmax(wf, blocksize)
    codes = encode(wf, a, thr, blocksize, order=order, zero_code=zero_code)
    out = {
        "quant_type": quant_type,
        "n": wf.size,
        "blocksize": blocksize,
        "double_quant": bool(double_quant_on),
        "group": group,
        "codes": codes,
        "packed": pack_nibbles(codes),
        "absmax_fp32": a,
    }
    if double_quant_on:
        if dq_map == "dynamic":
            q, s, mean = double_quant_dynamic(a, group)
        elif dq_map == "linear":
            q, s, mean = double_quant(a, group)
        else:
            raise ValueError(f"unknown second-level map {dq_map!r}")
        out.update(absmax=q, absmax2=s, absmax_mean=mean, dq_map=dq_map)
    else:
        out.update(absmax=a, absmax2=None, absmax_mean=None)
    return out


# --------------------------------------------------------------------------
# Step 6: dequantize to bfloat16
# --------------------------------------------------------------------------
def dequantize(packed: np.ndarray, state: dict, n: int | None = None,
               dtype: str = "bf16") -> np.ndarray:
    """W_hat_j = rnd(fl32(L[c_j] * a_hat_b)) as 16-bit patterns of the compute
    dtype, rnd = round to nearest even into BF16 or FP16 (section 3.4:
    dequantize back to the 16-bit compute dtype; section 4: BF16 or FP16).
    L is the level of each code for the state's quant type."""
    codes = unpack_nibbles(packed)
    if n is None:
        n = codes.size
    codes = codes[:n]
    levels = levels_by_code(state.get("quant_type", "nf4"))
    blocksize = state.get("blocksize", BLOCKSIZE)
    scale = block_scales(state)
    b = np.arange(n) // blocksize
    v = (levels[codes] * scale[b]).astype(np.float32)
    return f32_to_bits(v, dtype)


# --------------------------------------------------------------------------
# Step 7/8: the 4-bit-storage / 16-bit-compute linear layer
# --------------------------------------------------------------------------
def matmul_ref(x_bits: np.ndarray, w_bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Y = X . W^T in binary64 (nn.Linear orientation, no bias; pomoai.com
    overview, Linear4bit replacing torch.nn.Linear).  X is [M, K], W is
    [N, K], both 16-bit patterns of the compute dtype; the result is float64
    [M, N].  Library primitive: NumPy's binary64 matmul."""
    x = bits_to_f32(x_bits, dtype).astype(np.float64)
    w = bits_to_f32(w_bits, dtype).astype(np.float64)
    return x @ w.T


def dequant_matmul_ref(x_bits: np.ndarray, packed: np.ndarray, state: dict,
                       N: int, K: int, dtype: str = "bf16") -> np.ndarray:
    """The reference the dequant-GEMV/GEMM is compared to: dequantize the
    4-bit weight to the compute dtype (step 6), then multiply in binary64."""
    w_hat = dequantize(packed, state, N * K, dtype).reshape(N, K)
    return matmul_ref(np.asarray(x_bits).reshape(-1, K), w_hat, dtype)


def dequant_matmul_dx_ref(dy_bits: np.ndarray, packed: np.ndarray, state: dict,
                          N: int, K: int, dtype: str = "bf16") -> np.ndarray:
    """Input gradient of the layer above: dX = dY . W_hat for dY [M, N] and
    the dequantized weight W_hat [N, K] (step 6), in binary64.  The weight is
    frozen (the 4-bit base layer under QLoRA, pomoai.com overview), so this
    is the only gradient that flows through it.  Library primitive: NumPy's
    binary64 matmul."""
    w_hat = bits_to_f32(dequantize(packed, state, N * K, dtype), dtype).astype(np.float64)
    dy = bits_to_f32(np.asarray(dy_bits).reshape(-1, N), dtype).astype(np.float64)
    return dy @ w_hat.reshape(N, K)


def lora_matmul_ref(x_bits: np.ndarray, packed: np.ndarray, state: dict, N: int, K: int,
                    xa_bits: np.ndarray, b_bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """The 4-bit layer plus a low-rank adapter term (QLoRA, pomoai.com
    overview: adapters trained beside the frozen 4-bit base):
    Y = X . W_hat^T + XA . B^T with XA [M, r] (the scaled down-projection) and
    B [N, r] (the up-projection), in binary64."""
    r = np.asarray(b_bits).reshape(N, -1).shape[1]
    xa = bits_to_f32(np.asarray(xa_bits).reshape(-1, r), dtype).astype(np.float64)
    b = bits_to_f32(np.asarray(b_bits).reshape(N, r), dtype).astype(np.float64)
    return dequant_matmul_ref(x_bits, packed, state, N, K, dtype) + xa @ b.T


def lora_down_ref(x_bits: np.ndarray, a_bits: np.ndarray, scale: float, M: int, K: int,
                  dtype: str = "bf16") -> np.ndarray:
    """The adapter's scaled down-projection XA = s . X . A^T (QLoRA, pomoai.com
    overview: low-rank adapters beside the frozen 4-bit base; A [r, K] is the
    nn.Linear(K, r) weight, s the adapter's scale), X [M, K] and A in the
    compute dtype, in binary64 (no rounding).  Library primitive: NumPy's
    binary64 matmul."""
    x = bits_to_f32(np.asarray(x_bits).reshape(M, K), dtype).astype(np.float64)
    a = bits_to_f32(np.asarray(a_bits).reshape(-1, K), dtype).astype(np.float64)
    return float(scale) * (x @ a.T)


def rel_frobenius(y, y_ref) -> float:
    """||y - y_ref||_F / ||y_ref||_F in binary64."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(r)
    num = np.linalg.norm(y - r)
    return float(num / den) if den > 0 else float(num)


# --------------------------------------------------------------------------
# Memory arithmetic
# --------------------------------------------------------------------------
def storage_bytes(n: int, double_quant_on: bool, blocksize: int = BLOCKSIZE,
                  group: int = DQ_GROUP) -> int:
    """Bytes a quantized tensor of n weights occupies: n/2 of packed codes,
    plus FP32 scales per block (section 3.3, ordinary quantization), or int8
    scales per block + FP32 per group + the FP32 mean (double quantization)."""
    nb = _blocks(n, blocksize)
    if not double_quant_on:
        return n // 2 + 4 * nb
    return n // 2 + nb + 4 * _blocks(nb, group) + 4
