"""Plain CPU oracle for one MoE layer's routed-expert computation (fp64).

TEST INFRASTRUCTURE.  Only the tests (tests/), the smoke check in
__graft_entry__.smoke() and the cpu_baseline leg of bench.py may import or call
this module.  The product path (the HIP library and its Python binding) never
does, and this module imports nothing from it.

What it computes, step by step, and where each step is defined:

  Pages cited (title, site, date):
    [Strata]    "strata-expert-paths", hanayo.cn, 2026-10-13.
    [FreeToken] "FreeToken 阅读笔记" (FreeToken reading notes), zhongzhuzhou.org,
                2026-08-23.
    [PLE]       "【Qwen3.8-Flash-Next 端侧部署】02-PLE 如何从 NVMe 送到 GPU",
                mengman.github.io, 2026-09-10.

  1. Weight decode — [PLE] section "NVFP4 code 和 scale 如何反量化": the low and
     high nibble of a byte are two codes; a code's low 3 bits pick a magnitude
     from {0, .5, 1, 1.5, 2, 3, 4, 6} and its top bit is the sign; each run of
     16 values is multiplied by its FP8 E4M3 block scale and then by one FP32
     global scale.  E4M3 here is the OCP E4M3FN encoding (bias 7, subnormals,
     no infinity, S.1111.111 is NaN).  The product is exact in fp64.
  2. Router logits — [Strata] "显存里缓存的是什么？": the router decides which
     experts a token uses and the merge weight of each output.  When the router
     matrix is given, logits are x . W_r summed in fp64 and stored as fp32
     (rounding point R0); otherwise the logits are an input.
  3. Top-k — experts ordered by (logit descending, expert index ascending); the
     first k are slots 0..k-1 ([Strata] "还有一条会改变输出的路径" ranks a token's
     experts; ties to the lower index is the reading adopted).
  4. Weights — the softmax over all E logits renormalised to the k chosen:
     w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), in fp64.
  5. Shared gate — sigma_t = 1 / (1 + exp(-x_t . w_sg)) in fp64 ([Strata]
     "路由以后，专家怎样分工？": the gated shared-expert contribution).
  6. Groups — [Strata] "路由以后，专家怎样分工？": the tokens of a layer that picked
     the same expert form one group recording their inputs and output
     positions.  Groups in ascending expert index, rows inside a group in
     ascending token order; the shared expert's group is every token, last.
  7. Expert FFN per row — [Strata] "CPU 怎样把剩下的专家算完？": gate/up, the
     activation, the intermediate re-encoded for the next kernel, then down.
     g = Wg x, u = Wu x (fp64); h = bf16(g / (1 + e^-g) * u) (rounding point R1);
     Y = bf16(Wd h) (rounding point R3).
  8. Combine — [Strata] "路由以后，专家怎样分工？" and "少算这些专家，会付出什么代价？":
     y_t = bf16( sum_j w_j Y[row(t, j)] + sigma_t Y_shared[t] ) (rounding point
     R2), with no renormalisation.
  10. Partial residency (a variant) — [FreeToken] 3.3: one LRU cache over
     (layer, expert) shared by all layers; a hit refreshes the expert's last
     use, a fill admits a newly chosen expert, eviction removes the least
     recently used; and 4: per layer one step on the device dedups the routed
     experts, classifies them against the residency table, picks the victims
     (the least recently used slots, found in one pass) and rewrites the
     table.  Readings: every miss is filled; the clock ticks once per layer
     call; among slots of equal last use the lower slot index goes first;
     empty slots count as never used; the shared expert is always needed.
  11. Hot/cold swaps (a variant) — [Strata] "哪些专家能长期留在显存？" (the
     passages on heat and candidate pairs, and on swaps and publication): each
     expert's heat accumulates its routing counts; per round, inside one layer
     the hottest experts outside the cache pair with the coldest inside, a pair
     whose heat gap reaches the threshold (default 1.5) is a swap candidate,
     the candidates go by gap, at most 96 a round (default), and afterwards
     every heat is multiplied by the decay 0.7.  Readings: pairs are formed in
     order (i-th hottest outside with i-th coldest inside, ties to the lower
     expert index) and stop at the first pair below the threshold; the shared
     expert never swaps; equal gaps go by (layer, pair index); heats are fp32
     as on the device, so every comparison is taken in fp32.
  12. MX formats (a variant) — [FreeToken] notes that the DeepSeek-V4-Flash
     experts are natively MXFP4; the pages do not define the format, so the
     OCP Microscaling (MX) definitions are the reading adopted: 32 values along
     K share one E8M0 scale 2^(b - 127) (b = 255 is NaN); MXFP4 elements are
     E2M1 (no global scale); activations meet the scaled MFMA as MXFP8
     (elements E4M3FN), a new rounding point RA: per 32 values the shared
     exponent is floor(log2 amax) - 8 (clamped to [-127, 127]; a zero block
     takes -127) and each element is v / 2^shared rounded to the nearest
     E4M3FN value (ties to the even code), saturating at +-448.  The MX expert
     FFN quantises x at RA, rounds h to bf16 (R1) and quantises that at RA
     for the down projection.
  9. Route tail-skip (a variant) — [Strata] "少算这些专家，会付出什么代价？" and the
     skip-condition passage just before it: with a rank threshold R (default 7,
     ranks counted from zero), an expert that is not resident is skipped when
     every token of the window that picked it ranks it R or later.  A skipped
     expert's rows are zero and the kept weights are not renormalised, so the
     output moves by exactly -sum of the skipped w_i E_i(x).

bf16 rounding is round-to-nearest-even from the exact fp64 value (no detour
through fp32).  Parity pins for every function live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# 1. Formats
# ---------------------------------------------------------------------------

#: E2M1 magnitudes indexed by the low three bits of a code ([PLE], NVFP4 dequant).
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 nibble codes (0..15) -> fp64 values.  Bit 3 is the sign."""
    c = np.asarray(codes, dtype=np.int64)
    mag = np.asarray(E2M1_MAGNITUDES, dtype=np.float64)[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e4m3fn_decode(b) -> np.ndarray:
    """OCP FP8 E4M3FN bytes -> fp64.

    sign = bit 7, exponent = bits 3..6 (bias 7), mantissa = bits 0..2.
    exponent 0: subnormal m/8 * 2^-6; exponent 1..15: (1 + m/8) * 2^(e-7);
    exponent 15 with mantissa 7 is NaN; there is no infinity.
    """
    b = np.asarray(b, dtype=np.int64)
    s = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    sub = m / 8.0 * 2.0 ** -6
    norm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    v = s * np.where(e == 0, sub, norm)
    return np.where((e == 15) & (m == 7), np.nan, v)


@dataclass(frozen=True)
class BlobLayout:
    """Byte layout of one (layer, expert) blob, as specified in include/moe.h.

    Sections, each starting on a 256-byte boundary: gate codes (I x H/2 bytes),
    up codes, down codes (H x I/2), gate scales (I x H/16), up scales, down
    scales (H x I/16), then 3 fp32 globals (gate, up, down).  Inside a section
    the rows are tiled in blocks of 16 (see matrix_codes / matrix_scales).
    """

    H: int
    I: int
    off_codes: tuple
    off_scales: tuple
    off_globals: int
    blob_bytes: int
    slot_stride: int

    def matrix_shape(self, m: int):
        """(rows, K) of matrix m: 0 gate [I,H], 1 up [I,H], 2 down [H,I]."""
        return (self.I, self.H) if m < 2 else (self.H, self.I)


def _align(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def matrix_bytes(rows: int, K: int):
    """(code bytes, scale bytes) of one NVFP4 matrix: two codes per byte, one
    E4M3 scale per 16 values ([PLE] "一个 160 维向量在 packed 文件中占 90 字节")."""
    assert K % 16 == 0
    return rows * K // 2, rows * K // 16


def blob_layout(H: int, I: int) -> BlobLayout:
    shapes = [(I, H), (I, H), (H, I)]
    off = 0
    oc, os_ = [], []
    for r, K in shapes:
        oc.append(off)
        off = _align(off + matrix_bytes(r, K)[0], 256)
    for r, K in shapes:
        os_.append(off)
        off = _align(off + matrix_bytes(r, K)[1], 256)
    og = off
    blob = og + 12
    return BlobLayout(H, I, tuple(oc), tuple(os_), og, blob, _align(blob, 4096))


def _blob_bytes(blob) -> np.ndarray:
    return np.frombuffer(blob, dtype=np.uint8) if not isinstance(blob, np.ndarray) else blob.view(np.uint8)


def matrix_codes(blob, lay: BlobLayout, m: int) -> np.ndarray:
    """Code bytes of matrix m in row order, uint8 [rows, K/2] (byte c of a row:
    columns 2c, 2c+1).  Stored layout (include/moe.h): blocks of 16 rows, each
    8K bytes; inside a block the 32-column chunks follow one another, and a
    chunk holds the 16 rows' 16 bytes for it in row order."""
    rows, K = lay.matrix_shape(m)
    raw = _blob_bytes(blob)[lay.off_codes[m]: lay.off_codes[m] + matrix_bytes(rows, K)[0]]
    t = raw.reshape(rows // 16, K // 32, 16, 16)          # [block][chunk][row in block][byte]
    return t.transpose(0, 2, 1, 3).reshape(rows, K // 2)


def matrix_scales(blob, lay: BlobLayout, m: int) -> np.ndarray:
    """E4M3 scale bytes of matrix m in row order, uint8 [rows, K/16] (scale b:
    columns 16b..16b+15).  Stored layout (include/moe.h): blocks of 16 rows,
    each K bytes; inside a block the columns form groups of 512 (the last may
    be shorter), and a group holds each row's scales for it, rows in order."""
    rows, K = lay.matrix_shape(m)
    raw = _blob_bytes(blob)[lay.off_scales[m]: lay.off_scales[m] + matrix_bytes(rows, K)[1]]
    blocks = raw.reshape(rows // 16, K)
    out = np.empty((rows, K // 16), dtype=np.uint8)
    for g0 in range(0, K // 16, 32):                       # 32 scales per row per group
        n = min(32, K // 16 - g0)
        grp = blocks[:, 16 * g0: 16 * g0 + 16 * n].reshape(rows // 16, 16, n)
        out[:, g0: g0 + n] = grp.reshape(rows, n)
    return out


def dequant(blob, lay: BlobLayout, m: int) -> np.ndarray:
    """Matrix m of a blob as exact fp64 [rows, K]:
    value(r, c) = e2m1(code(r, c)) * e4m3(scale(r, c // 16)) * global."""
    buf = _blob_bytes(blob)
    rows, K = lay.matrix_shape(m)
    codes = matrix_codes(blob, lay, m)
    scales = matrix_scales(blob, lay, m)
    g = float(np.frombuffer(buf[lay.off_globals + 4 * m: lay.off_globals + 4 * m + 4].tobytes(), dtype="<f4")[0])
    q = np.empty((rows, K), dtype=np.float64)
    q[:, 0::2] = e2m1_decode(codes & 0xF)          # even column: low nibble
    q[:, 1::2] = e2m1_decode(codes >> 4)           # odd column: high nibble
    s = e4m3fn_decode(scales)                      # [rows, K/16]
    return q * np.repeat(s, 16, axis=1) * g


# ---------------------------------------------------------------------------
# Rounding points
# ---------------------------------------------------------------------------

_BF16_OVERFLOW = 2.0 ** 128


def bf16_round(v) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value, ties to even, directly
    from the fp64 value.  Returns fp64 holding bf16-representable values."""
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    fin = np.isfinite(v) & (v != 0)
    _, e = np.frexp(v[fin])                        # v = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)                    # 8 significant bits; subnormal quantum 2^-133
    r = np.ldexp(np.rint(np.ldexp(v[fin], -q)), q)  # np.rint: round half to even
    r = np.where(np.abs(r) >= _BF16_OVERFLOW, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """fp64 -> bf16 bit patterns, rounding to nearest even."""
    r = bf16_round(v).astype(np.float32)            # exact: r is on the bf16 grid
    return (r.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# 2-5. Router
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """logits[t, e] = fp32( sum_h x[t, h] * W_r[h, e] ), summed in fp64 (R0)."""
    return (np.asarray(x, np.float64) @ np.asarray(w_router, np.float64)).astype(np.float32)


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per row; ties go to the lower index.
    Slot j holds the j-th in order (logit descending, index ascending)."""
    lg = np.asarray(logits, dtype=np.float64)
    assert np.all(np.isfinite(lg)), "logits must be finite"
    order = np.argsort(-lg, axis=1, kind="stable")  # stable: equal keys keep index order
    return order[:, :k].astype(np.int32)


def topk_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0) over the chosen k (fp64)."""
    lg = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(lg, np.asarray(ids, np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    return ex / ex.sum(axis=1, keepdims=True)


def shared_gate(x: np.ndarray, w_shared_gate: np.ndarray) -> np.ndarray:
    """sigma_t = 1 / (1 + exp(-x_t . w_sg)) in fp64."""
    z = np.asarray(x, np.float64) @ np.asarray(w_shared_gate, np.float64)
    return 1.0 / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------
# 6. Grouping
# ---------------------------------------------------------------------------

@dataclass
class Groups:
    offsets: np.ndarray   # int32 [E+2]
    perm: np.ndarray      # int32 [T*k]: row p -> flat index f = t*k + j
    inv_perm: np.ndarray  # int32 [T*k]: f -> p


def group(ids: np.ndarray, E: int) -> Groups:
    """For e = 0..E-1 in order, append the flat rows f = t*k + j with
    ids[t, j] == e, t ascending.  The shared group (index E) is rows
    [T*k, T*k + T) in token order."""
    T, k = ids.shape
    flat = np.asarray(ids, np.int64).reshape(-1)
    perm: List[int] = []
    offsets = np.zeros(E + 2, dtype=np.int32)
    for e in range(E):
        offsets[e] = len(perm)
        perm.extend(np.nonzero(flat == e)[0].tolist())   # ascending f == ascending t
    offsets[E] = len(perm)
    offsets[E + 1] = T * k + T
    assert len(perm) == T * k, "every id must lie in [0, E)"
    perm_a = np.asarray(perm, dtype=np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    inv[perm_a] = np.arange(T * k, dtype=np.int32)
    return Groups(offsets, perm_a, inv)


# ---------------------------------------------------------------------------
# 7. Expert FFN
# ---------------------------------------------------------------------------

@dataclass
class FfnRows:
    h_pre: np.ndarray   # fp64 [n, I], before R1
    h: np.ndarray       # fp64 [n, I], bf16 values (R1)
    y_pre: np.ndarray   # fp64 [n, H], before R3
    y: np.ndarray       # fp64 [n, H], bf16 values (R3)


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def expert_ffn(x_rows: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> FfnRows:
    """Rows of one expert: h = bf16(silu(Wg x) * (Wu x)); Y = bf16(Wd h)."""
    xr = np.asarray(x_rows, np.float64)
    g = xr @ wg.T
    u = xr @ wu.T
    h_pre = silu(g) * u
    h = bf16_round(h_pre)
    y_pre = h @ wd.T
    return FfnRows(h_pre, h, y_pre, bf16_round(y_pre))


# ---------------------------------------------------------------------------
# 8. Combine
# ---------------------------------------------------------------------------

def combine(y_routed: np.ndarray, w: np.ndarray, sigma: np.ndarray, y_shared: np.ndarray):
    """y_t = bf16( sum_j w[t,j] * y_routed[t,j,:] + sigma_t * y_shared[t,:] ).

    y_routed: fp64 [n, k, H], the bf16 expert rows of each token's slots in slot
    order; y_shared: fp64 [n, H].  Returns (fp64 sum before R2, bf16-rounded)."""
    acc = np.zeros(y_shared.shape, dtype=np.float64)
    for j in range(y_routed.shape[1]):
        acc = acc + w[:, j:j + 1] * y_routed[:, j, :]
    acc = acc + sigma[:, None] * y_shared
    return acc, bf16_round(acc)


# ---------------------------------------------------------------------------
# 9. Route tail-skip (variant)
# ---------------------------------------------------------------------------

def tail_skip(ids: np.ndarray, resident: np.ndarray, skip_rank: int) -> np.ndarray:
    """The experts one window skips (bool [E]).

    ids: int [T, k] of the window's tokens (slot j = rank j, from zero);
    resident: bool [E].  Expert e is skipped when it is not resident, some token
    picked it, and every token that picked it ranks it at skip_rank or later.
    A single token ranking it earlier keeps it; a resident expert is always
    kept; skip_rank <= 0 skips nothing."""
    ids = np.asarray(ids)
    E = len(resident)
    out = np.zeros(E, dtype=bool)
    if skip_rank <= 0:
        return out
    for e in range(E):
        if resident[e]:
            continue
        ranks = [j for t in range(ids.shape[0]) for j in range(ids.shape[1]) if ids[t, j] == e]
        out[e] = len(ranks) > 0 and min(ranks) >= skip_rank
    return out


# ---------------------------------------------------------------------------
# 10. Partial residency (variant)
# ---------------------------------------------------------------------------

class LruCache:
    """S device slots caching (layer, expert) blobs; key = layer * (E + 1) + e.

    slot_table [L][E+1] (slot or -1), owner [S] (key or -1), last [S] (clock
    of the last use, -1 for a slot never used) and the clock, as the device
    keeps them."""

    def __init__(self, L: int, E: int, S: int):
        self.L, self.E, self.S = L, E, S
        self.slot_table = np.full((L, E + 1), -1, np.int32)
        self.owner = np.full(S, -1, np.int32)
        self.last = np.full(S, -1, np.int32)
        self.clock = 0

    def step(self, layer: int, ids: np.ndarray):
        """One layer call of the window `ids` [T, k].  Returns (fills, full):
        fills lists (key, slot) in the order the misses were placed; full is
        True when there were more misses than slots to evict (the misses past
        the available slots stay non-resident)."""
        E1 = self.E + 1
        now = self.clock
        self.clock += 1
        needed = sorted({int(e) for e in np.asarray(ids).ravel() if 0 <= e < self.E} | {self.E})
        for e in needed:                          # hits refresh their last use
            s = int(self.slot_table[layer, e])
            if s >= 0:
                self.last[s] = now
        misses = [e for e in needed if self.slot_table[layer, e] < 0]
        # victims: the least recently used slots; this call's hits (last == now)
        # are not candidates
        cand = sorted((int(self.last[s]), s) for s in range(self.S) if self.last[s] != now)
        full = len(misses) > len(cand)
        fills = []
        for e, (_, s) in zip(misses, cand):
            old = int(self.owner[s])
            if old >= 0:
                self.slot_table[old // E1, old % E1] = -1
            key = layer * E1 + e
            self.owner[s] = key
            self.last[s] = now
            self.slot_table[layer, e] = s
            fills.append((key, s))
        return fills, full


# ---------------------------------------------------------------------------
# 11. Hot/cold swaps (variant)
# ---------------------------------------------------------------------------

def heat_add(heat: np.ndarray, layer: int, ids: np.ndarray) -> None:
    """heat [L][E] fp32 += routing counts of the window ids [T, k] (ids outside
    [0, E) are not counted)."""
    E = heat.shape[1]
    counts = np.zeros(E, np.float32)
    for e in np.asarray(ids).ravel():
        if 0 <= e < E:
            counts[e] += np.float32(1.0)
    heat[layer] = (heat[layer] + counts).astype(np.float32)


def heat_decay(heat: np.ndarray, decay: float = 0.7) -> None:
    """Every heat times the decay, in fp32."""
    heat[...] = (heat * np.float32(decay)).astype(np.float32)


def swap_plan(heat: np.ndarray, slot_table: np.ndarray, threshold: float = 1.5, max_swaps: int = 96):
    """The round's swaps: a list of (layer, hot expert, cold expert), largest
    heat gap first.  heat [L][E] fp32; slot_table [L][E+1] (-1: not resident;
    column E, the shared expert, never swaps)."""
    L, E = heat.shape
    thr = np.float32(threshold)
    cands = []
    for l in range(L):
        out = sorted((e for e in range(E) if slot_table[l, e] < 0), key=lambda e: (-heat[l, e], e))
        ins = sorted((e for e in range(E) if slot_table[l, e] >= 0), key=lambda e: (heat[l, e], e))
        for i in range(min(len(out), len(ins))):
            gap = np.float32(heat[l, out[i]] - heat[l, ins[i]])
            if not gap >= thr:
                break
            cands.append((-gap, l, i, out[i], ins[i]))
    cands.sort()
    return [(l, hot, cold) for _, l, _, hot, cold in cands[:max_swaps]]


# ---------------------------------------------------------------------------
# 12. MX formats (variant)
# ---------------------------------------------------------------------------

def e8m0_decode(b) -> np.ndarray:
    """E8M0 scale bytes -> 2^(b - 127); 255 is NaN."""
    b = np.asarray(b, dtype=np.int64)
    return np.where(b == 255, np.nan, np.exp2(b.astype(np.float64) - 127.0))


def _e4m3_table():
    codes = np.array([c for c in range(128) if c != 0x7F], dtype=np.int64)   # non-negative finite codes
    vals = e4m3fn_decode(codes)
    order = np.argsort(vals, kind="stable")
    return vals[order], codes[order]


_E4M3_VALS, _E4M3_CODES = _e4m3_table()


def e4m3fn_encode(v) -> np.ndarray:
    """fp64 -> OCP E4M3FN bytes: the nearest representable value, ties to the
    even code (even mantissa), saturating at +-448; -0 encodes as 0x80."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    i = np.clip(np.searchsorted(_E4M3_VALS, a), 1, len(_E4M3_VALS) - 1)
    lo, hi = _E4M3_VALS[i - 1], _E4M3_VALS[i]
    clo, chi = _E4M3_CODES[i - 1], _E4M3_CODES[i]
    pick_hi = (hi - a < a - lo) | ((hi - a == a - lo) & ((chi & 1) == 0))
    code = np.where(a >= hi, chi, np.where(pick_hi, chi, clo))
    code = np.where(a <= 0.0, 0, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def mxfp8_quantize(v: np.ndarray):
    """Rows of v [n, K] (K % 32 == 0) at rounding point RA.  Returns (E4M3
    codes uint8 [n, K], E8M0 scale bytes uint8 [n, K/32], fp64 values)."""
    v = np.asarray(v, dtype=np.float64)
    n, K = v.shape
    blocks = v.reshape(n, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))       # amax = m 2^ex, 0.5 <= m < 1
    shared = np.where(amax > 0, np.clip(ex - 1 - 8, -127, 127), -127)
    X = np.exp2(shared.astype(np.float64))[:, :, None]
    codes = e4m3fn_encode(blocks / X)
    vals = e4m3fn_decode(codes) * X
    return codes.reshape(n, K), (shared + 127).astype(np.uint8), vals.reshape(n, K)


@dataclass
class MxBlobLayout:
    blob_bytes: int
    slot_stride: int
    off_codes: tuple
    off_scales: tuple


def mx_blob_layout(H: int, I: int) -> MxBlobLayout:
    """MXFP4 blob: gate, up, down codes (the NVFP4 blob's placement), then their
    E8M0 scales; no global scales.  Scale placement: per 16-row block, K/2
    bytes; inside it group g of four 32-value blocks takes 64 bytes, row r's
    four bytes at 4 r (so the scale byte of (row n, block b) sits at
    (n // 16) * (K / 2) + (b // 4) * 64 + (n % 16) * 4 + b % 4).  Needs K % 128
    == 0 and rows % 16 == 0."""
    assert H % 128 == 0 and I % 128 == 0
    rows = (I, I, H)
    ks = (H, H, I)
    off = 0
    oc, osc = [], []
    for r, K in zip(rows, ks):
        oc.append(off)
        off = _align(off + r * K // 2, 256)
    for r, K in zip(rows, ks):
        osc.append(off)
        off = _align(off + r * K // 32, 256)
    return MxBlobLayout(off, _align(off, 4096), tuple(oc), tuple(osc))


def mx_matrix_scales(blob, lay: MxBlobLayout, m: int, H: int, I: int) -> np.ndarray:
    """E8M0 scale bytes of matrix m as [rows][K/32]."""
    rows, K = ((I, H), (I, H), (H, I))[m]
    b = _blob_bytes(blob)
    raw = b[lay.off_scales[m]:lay.off_scales[m] + rows * K // 32]
    # [row block][group][row in block][block in group]
    t = raw.reshape(rows // 16, K // 128, 16, 4)
    return t.transpose(0, 2, 1, 3).reshape(rows, K // 32)


def mx_dequant(blob, lay: MxBlobLayout, m: int, H: int, I: int) -> np.ndarray:
    """Matrix m as fp64 [rows][K]: e2m1(code) * 2^(scale - 127).  Exact."""
    rows, K = ((I, H), (I, H), (H, I))[m]
    nv = BlobLayout(H, I, lay.off_codes, lay.off_scales, 0, lay.blob_bytes, lay.slot_stride)
    codes = matrix_codes(blob, nv, m)
    q = np.empty((rows, K), dtype=np.float64)
    q[:, 0::2] = e2m1_decode(codes & 0xF)          # even column: low nibble
    q[:, 1::2] = e2m1_decode(codes >> 4)
    sc = e8m0_decode(mx_matrix_scales(blob, lay, m, H, I))
    return q * np.repeat(sc, 32, axis=1)


def expert_ffn_mx(x_rows: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> FfnRows:
    """The MX expert FFN: x at RA, gate/up, h = bf16(silu(g) u) (R1), h at RA,
    down, Y = bf16(o) (R3).  Weights are the exact MX dequantisation."""
    xq = mxfp8_quantize(x_rows)[2]
    g = xq @ wg.T
    u = xq @ wu.T
    h_pre = silu(g) * u
    h = bf16_round(h_pre)
    y_pre, y = down_mx(h, wd)
    return FfnRows(h_pre, h, y_pre, y)


def down_mx(h: np.ndarray, wd: np.ndarray):
    """The MX FFN from bf16 rows h on: h at RA, the down projection, Y = bf16(o)
    (R3).  Returns (Y before R3, Y)."""
    hq = mxfp8_quantize(h)[2]
    y_pre = hq @ wd.T
    return y_pre, bf16_round(y_pre)


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

@dataclass
class LayerResult:
    logits: np.ndarray          # fp32 [T, E]
    ids: np.ndarray             # int32 [T, k]
    w: np.ndarray               # fp64 [T, k]
    sigma: np.ndarray           # fp64 [T]
    groups: Groups
    tokens: np.ndarray          # int64 [n]: tokens whose rows/outputs were computed
    h: Dict[int, np.ndarray] = field(default_factory=dict)      # row p -> fp64 [I] (bf16 values)
    h_pre: Dict[int, np.ndarray] = field(default_factory=dict)
    y_rows: Dict[int, np.ndarray] = field(default_factory=dict)  # row p -> fp64 [H] (bf16 values)
    y_rows_pre: Dict[int, np.ndarray] = field(default_factory=dict)
    y_pre: Optional[np.ndarray] = None   # fp64 [n, H] before R2
    y: Optional[np.ndarray] = None       # fp64 [n, H] bf16 values


def moe_layer(x_bits: np.ndarray, blob_of: Callable[[int], bytes], H: int, I: int, E: int, k: int,
              w_shared_gate: np.ndarray, w_router: Optional[np.ndarray] = None,
              logits: Optional[np.ndarray] = None, tokens: Optional[Sequence[int]] = None,
              dense_weights: Optional[Dict[int, tuple]] = None,
              skip: Optional[np.ndarray] = None, fmt: str = "nvfp4") -> LayerResult:
    """One MoE layer.

    x_bits: uint16 bf16 bits [T, H].  blob_of(e) returns the blob bytes of
    expert e (e == E is the shared expert).  Exactly one of w_router / logits.
    Routing and grouping cover every token; the FFN rows and the combine are
    computed for `tokens` (default: all), since a token's output depends only
    on its own row, its routing and the expert bytes.  skip (bool [E], see
    tail_skip): the routed rows of a skipped expert are zero (h and Y), so its
    terms drop out of the combine and the other weights stay as they are.
    fmt "mx": the blobs are MXFP4 (mx_blob_layout) and each expert runs
    expert_ffn_mx.
    """
    assert (w_router is None) != (logits is None)
    T = x_bits.shape[0]
    x = bf16_bits_to_f64(x_bits)
    lg = router_logits(x, w_router) if w_router is not None else np.asarray(logits, np.float32)
    ids = topk(lg, k)
    w = topk_weights(lg, ids)
    sigma = shared_gate(x, w_shared_gate)
    groups = group(ids, E)
    tok = np.arange(T) if tokens is None else np.asarray(sorted(set(int(t) for t in tokens)), np.int64)
    res = LayerResult(lg, ids, w, sigma, groups, tok)

    assert fmt in ("nvfp4", "mx")
    lay = blob_layout(H, I) if fmt == "nvfp4" else mx_blob_layout(H, I)
    cache = {} if dense_weights is None else dense_weights
    ffn = expert_ffn if fmt == "nvfp4" else expert_ffn_mx

    def weights(e):
        if e not in cache:
            b = blob_of(e)
            cache[e] = tuple(dequant(b, lay, m) if fmt == "nvfp4" else mx_dequant(b, lay, m, H, I)
                             for m in range(3))
        return cache[e]

    # rows needed, grouped by expert: (expert, row p, token t)
    need: Dict[int, List[tuple]] = {}
    for t in tok:
        for j in range(k):
            f = int(t) * k + j
            need.setdefault(int(ids[t, j]), []).append((int(groups.inv_perm[f]), int(t)))
        need.setdefault(E, []).append((T * k + int(t), int(t)))
    for e in sorted(need):
        rows = need[e]
        if skip is not None and e < E and skip[e]:
            for p, _ in rows:
                res.h_pre[p] = res.h[p] = np.zeros(I)
                res.y_rows_pre[p] = res.y_rows[p] = np.zeros(H)
            continue
        wg, wu, wd = weights(e)
        out = ffn(x[[t for _, t in rows]], wg, wu, wd)
        for i, (p, _) in enumerate(rows):
            res.h_pre[p], res.h[p] = out.h_pre[i], out.h[i]
            res.y_rows_pre[p], res.y_rows[p] = out.y_pre[i], out.y[i]
        if dense_weights is None:
            cache.pop(e, None)   # keep memory bounded for large experts

    yr = np.stack([np.stack([res.y_rows[int(groups.inv_perm[int(t) * k + j])] for j in range(k)]) for t in tok])
    ysh = np.stack([res.y_rows[T * k + int(t)] for t in tok])
    res.y_pre, res.y = combine(yr, w[tok], sigma[tok], ysh)
    return res
