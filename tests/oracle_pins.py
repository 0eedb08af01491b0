"""Pins for the fp64 oracle: facts about attention that do not come from the
oracle itself.

Each check takes a loaded oracle build and raises AssertionError when the
build disagrees with
  - the IEEE 754 definitions of the storage types (and numpy's own fp16),
  - a brute-force evaluation of the definition in 40-digit decimal
    arithmetic on tiny inputs, without the max-subtraction the oracle uses,
  - PyTorch's CPU scaled_dot_product_attention in float64 (a library
    routine for the same definition),
  - closed forms (one key; two keys give logistic weights; a zero query or a
    zero scale gives the mean of V; constant V; identical keys; a very large
    scale picks V at the arg-max), and
  - invariants that hold for any input (softmax rows sum to one; joint K/V
    row permutation; Q row permutation; a common shift of all keys; linearity
    in V; the causal prefix property; heads are independent).

The definition checked is the one of "Android Transformer Optimization:
Attention and Mobile GPU Bottlenecks", section "The Self-Attention Bottleneck
Is Memory Traffic, Not Compute", with the softmax scale of "Flash Attention on
Android: tiled SGEMM with RenderScript", section "Architecture: tiled
attention with RenderScript BLAS".  The mutation tests run the same checks on
deliberately broken copies of the oracle and require that every copy fails at
least one of them.
"""

import math
from decimal import Decimal, getcontext

import numpy as np

from workloads import round_to_storage

DTYPES = ("f32", "f16", "bf16")


# ---------------------------------------------------------------- helpers --

def np_decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bits -> float64 by numpy's own conversions (independent of the
    oracle's decoders)."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
            return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
        with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
            return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def rand_bits(shape, dtype, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape) * sigma).astype(np.float32)
    return round_to_storage(x, dtype)


def dyadic_bits(shape, dtype, seed, lo=-8, hi=8, denom=4):
    """Values k/denom with small integers k: exact in every storage type, and
    sums of two of them stay exact."""
    rng = np.random.default_rng(seed)
    x = (rng.integers(lo, hi + 1, size=shape) / denom).astype(np.float32)
    return round_to_storage(x, dtype)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def brute_force(qf, kf, vf, scale, causal):
    """The definition in 40-digit decimal arithmetic, one (N, D) head.  The
    softmax is evaluated as exp(s_ij) / sum_j exp(s_ij) without subtracting
    the row maximum (decimal exponents do not overflow here)."""
    getcontext().prec = 40
    N, D = qf.shape
    sc = Decimal(float(scale))
    out = np.zeros((N, D))
    for i in range(N):
        w = []
        for j in range(N):
            if causal and j > i:
                w.append(Decimal(0))
                continue
            s = sum((Decimal(float(qf[i, d])) * Decimal(float(kf[j, d])) for d in range(D)),
                    Decimal(0))
            w.append((s * sc).exp())
        tot = sum(w, Decimal(0))
        for d in range(D):
            num = sum((w[j] * Decimal(float(vf[j, d])) for j in range(N)), Decimal(0))
            out[i, d] = float(num / tot)
    return out


# ----------------------------------------------------------------- checks --

def check_decode_known_values(orc):
    """Bit patterns whose values follow from the IEEE 754 binary16 and
    binary32 layouts (bf16 is the upper half of binary32)."""
    f16 = {0x0000: 0.0, 0x3C00: 1.0, 0xBC00: -1.0, 0x4000: 2.0, 0x3800: 0.5,
           0x7BFF: 65504.0, 0x0400: 2.0 ** -14, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
           0x3555: 0.333251953125, 0xC500: -5.0, 0x7C00: math.inf, 0xFC00: -math.inf}
    bf16 = {0x0000: 0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4049: 3.140625, 0x4000: 2.0,
            0x3F00: 0.5, 0x7F7F: 255 * 2.0 ** 120, 0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133,
            0xC0A0: -5.0, 0x7F80: math.inf, 0xFF80: -math.inf}
    f32 = {0x3F800000: 1.0, 0xC0A00000: -5.0, 0x00000001: 2.0 ** -149,
           0x7F7FFFFF: (2 - 2.0 ** -23) * 2.0 ** 127, 0x3EAAAAAB: 11184811 * 2.0 ** -25}
    for table, dtype in ((f16, "f16"), (bf16, "bf16")):
        bits = np.array(list(table), dtype=np.uint16)
        got = orc.decode(bits, dtype)
        assert list(got) == list(table.values()), f"{dtype} decode {got} != {list(table.values())}"
    bits = np.array(list(f32), dtype=np.uint32).view(np.float32)
    got = orc.decode(bits, "f32")
    assert list(got) == list(f32.values()), f"f32 decode {got}"
    nan = orc.decode(np.array([0x7E00], dtype=np.uint16), "f16")
    assert np.isnan(nan).all(), "f16 0x7E00 must decode to NaN"


def check_decode_all_16bit_patterns(orc):
    """Every fp16 pattern against numpy's float16, every bf16 pattern
    against the binary32 it is the upper half of."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dtype in ("f16", "bf16"):
        got = orc.decode(allbits, dtype)
        ref = np_decode(allbits, dtype)
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        bad = np.flatnonzero(~same)
        assert bad.size == 0, f"{dtype}: {bad.size} patterns differ, first 0x{int(allbits[bad[0]]):04X}"


def check_brute_force_decimal(orc):
    """Tiny heads in every storage type and both mask settings against the
    40-digit evaluation of the definition."""
    cases = [((1, 1, 1, 1), 1.0), ((1, 1, 2, 3), None), ((1, 2, 5, 4), None),
             ((2, 1, 8, 4), 0.9), ((1, 1, 7, 2), None)]
    seed = 11
    for dtype in DTYPES:
        for causal in (False, True):
            for shape, scale in cases:
                seed += 1
                q = rand_bits(shape, dtype, seed, 1.5)
                k = rand_bits(shape, dtype, seed + 1000, 1.5)
                v = rand_bits(shape, dtype, seed + 2000)
                sc = scale if scale is not None else 1.0 / math.sqrt(shape[3])
                got = orc.forward(q, k, v, dtype, sc, causal)
                qf, kf, vf = (np_decode(t, dtype) for t in (q, k, v))
                for b in range(shape[0]):
                    for h in range(shape[1]):
                        ref = brute_force(qf[b, h], kf[b, h], vf[b, h], sc, causal)
                        _close(got[b, h], ref, 1e-13,
                               f"brute force {dtype} causal={causal} shape={shape} head={b},{h}")


def check_torch_sdpa_fp64(orc):
    """Moderate sizes (several rows, ragged lengths, D = 64/96/128) against
    torch.nn.functional.scaled_dot_product_attention on float64 CPU
    tensors, whose causal mask also keeps key j <= query i."""
    import torch
    cases = [((1, 2, 129, 64), "f16", False), ((1, 2, 129, 64), "f16", True),
             ((2, 1, 100, 96), "bf16", True), ((1, 1, 64, 128), "f32", False),
             ((1, 1, 77, 128), "f32", True)]
    for idx, (shape, dtype, causal) in enumerate(cases):
        q = rand_bits(shape, dtype, 500 + idx, 2.0)
        k = rand_bits(shape, dtype, 600 + idx, 2.0)
        v = rand_bits(shape, dtype, 700 + idx)
        sc = 1.0 / math.sqrt(shape[3])
        got = orc.forward(q, k, v, dtype, sc, causal)
        qt, kt, vt = (torch.from_numpy(np_decode(t, dtype)) for t in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal,
                                                               scale=sc).numpy()
        _close(got, ref, 1e-12, f"torch sdpa {shape} {dtype} causal={causal}")


def check_single_key(orc):
    """N = 1: the only weight is 1, so O = V."""
    for dtype in DTYPES:
        for causal in (False, True):
            q, k, v = (rand_bits((2, 3, 1, 64), dtype, s) for s in (1, 2, 3))
            got = orc.forward(q, k, v, dtype, 0.125, causal)
            _close(got, np_decode(v, dtype), 0.0, f"N=1 {dtype} causal={causal}")


def check_two_keys_logistic(orc):
    """N = 2, non-causal: O_i = sigma(s_i0 - s_i1) V_0 + sigma(s_i1 - s_i0) V_1
    with sigma(x) = 1 / (1 + exp(-x)).  Causal row 0 is V_0 and causal row 1
    is the same logistic mix."""
    dtype = "f32"
    q, k, v = (rand_bits((1, 1, 2, 8), dtype, s, 1.3) for s in (21, 22, 23))
    qf, kf, vf = (np_decode(t, dtype)[0, 0] for t in (q, k, v))
    sc = 0.7
    for causal in (False, True):
        got = orc.forward(q, k, v, dtype, sc, causal)[0, 0]
        for i in range(2):
            s0 = sc * float(np.dot(qf[i], kf[0]))
            s1 = sc * float(np.dot(qf[i], kf[1]))
            if causal and i == 0:
                ref = vf[0]
            else:
                w0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
                w1 = 1.0 / (1.0 + math.exp(-(s1 - s0)))
                ref = w0 * vf[0] + w1 * vf[1]
            _close(got[i], ref, 1e-14, f"two keys causal={causal} row {i}")


def check_uniform_scores_mean(orc):
    """All scores of a row equal -> O_i is the mean of the visible V rows.
    Three ways to get there: Q = 0, scale = 0, and all K rows identical."""
    for dtype in DTYPES:
        shape = (1, 2, 37, 64)
        q = rand_bits(shape, dtype, 31)
        k = rand_bits(shape, dtype, 32)
        v = rand_bits(shape, dtype, 33)
        vf = np_decode(v, dtype)
        full_mean = np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape)
        prefix_mean = np.cumsum(vf, axis=2) / np.arange(1, shape[2] + 1)[None, None, :, None]
        zero_q = np.zeros_like(q)
        same_k = np.ascontiguousarray(np.broadcast_to(k[:, :, :1, :], k.shape))
        for causal, ref in ((False, full_mean), (True, prefix_mean)):
            _close(orc.forward(zero_q, k, v, dtype, 0.125, causal), ref, 1e-13,
                   f"Q=0 {dtype} causal={causal}")
            _close(orc.forward(q, k, v, dtype, 0.0, causal), ref, 1e-13,
                   f"scale=0 {dtype} causal={causal}")
            _close(orc.forward(q, same_k, v, dtype, 0.125, causal), ref, 1e-13,
                   f"identical K rows {dtype} causal={causal}")


def check_constant_v(orc):
    """Every V row the same vector c -> every O row is c (weights sum to 1)."""
    for dtype in DTYPES:
        shape = (2, 2, 45, 96)
        q = rand_bits(shape, dtype, 41, 2.0)
        k = rand_bits(shape, dtype, 42, 2.0)
        row = rand_bits((1, 1, 1, 96), dtype, 43)
        v = np.ascontiguousarray(np.broadcast_to(row, shape))
        for causal in (False, True):
            got = orc.forward(q, k, v, dtype, 0.1, causal)
            _close(got, np.broadcast_to(np_decode(row, dtype), shape), 1e-13,
                   f"constant V {dtype} causal={causal}")


def check_large_scale_argmax(orc):
    """A scale so large that the top score of a row beats the next by more
    than 60 (e^-60 ~ 1e-26) -> O_i = V[argmax_j s_ij].  Rows whose top two
    scores are closer are skipped.  The scaled scores reach ~1e3, so this
    also needs the max-subtraction: exp(1e3) overflows fp64."""
    dtype = "f32"
    shape = (1, 1, 50, 16)
    q, k, v = (rand_bits(shape, dtype, s) for s in (51, 52, 53))
    qf, kf, vf = (np_decode(t, dtype)[0, 0] for t in (q, k, v))
    sc = 300.0
    for causal in (False, True):
        got = orc.forward(q, k, v, dtype, sc, causal)[0, 0]
        s = sc * (qf @ kf.T)
        if causal:
            s = np.where(np.tril(np.ones_like(s)) > 0, s, -np.inf)
        checked = 0
        for i in range(shape[2]):
            top = np.sort(s[i][np.isfinite(s[i])])[::-1]
            if top.size > 1 and top[0] - top[1] < 60:
                continue
            checked += 1
            _close(got[i], vf[int(np.argmax(s[i]))], 1e-13, f"argmax row {i} causal={causal}")
        assert checked >= 10, "too few well-separated rows"


def check_rowsums_one(orc):
    """Each softmax row sums to one."""
    for dtype in DTYPES:
        for causal in (False, True):
            q, k, v = (rand_bits((1, 3, 65, 64), dtype, s, 3.0) for s in (61, 62, 63))
            _, rs, _ = orc.forward(q, k, v, dtype, 0.125, causal, return_rowsum=True)
            _close(rs, np.ones_like(rs), 1e-12, f"row sums {dtype} causal={causal}")


def check_kv_permutation(orc):
    """Non-causal attention does not depend on the order of the keys when K
    and V rows are permuted together."""
    for dtype in DTYPES:
        shape = (1, 2, 70, 64)
        q, k, v = (rand_bits(shape, dtype, s) for s in (71, 72, 73))
        perm = np.random.default_rng(74).permutation(shape[2])
        kp = np.ascontiguousarray(k[:, :, perm])
        vp = np.ascontiguousarray(v[:, :, perm])
        _close(orc.forward(q, kp, vp, dtype, 0.125, False), orc.forward(q, k, v, dtype, 0.125, False),
               1e-13, f"K/V permutation {dtype}")


def check_q_permutation(orc):
    """Non-causal attention is row-wise: permuting Q rows permutes O rows."""
    dtype = "f16"
    shape = (1, 2, 70, 64)
    q, k, v = (rand_bits(shape, dtype, s) for s in (81, 82, 83))
    perm = np.random.default_rng(84).permutation(shape[2])
    qp = np.ascontiguousarray(q[:, :, perm])
    base = orc.forward(q, k, v, dtype, 0.125, False)
    _close(orc.forward(qp, k, v, dtype, 0.125, False), base[:, :, perm], 1e-14, "Q permutation")


def check_key_shift(orc):
    """Adding one vector u to every key adds scale*<q_i, u> to every score of
    row i, which the softmax cancels.  Dyadic values keep K + u exact."""
    for dtype in DTYPES:
        shape = (1, 2, 40, 64)
        q = dyadic_bits(shape, dtype, 91)
        k = dyadic_bits(shape, dtype, 92)
        v = rand_bits(shape, dtype, 93)
        u = np.random.default_rng(94).integers(-8, 9, size=(1, 2, 1, 64)) / 4
        ks = round_to_storage((np_decode(k, dtype) + u).astype(np.float32), dtype)
        assert np.array_equal(np_decode(ks, dtype), np_decode(k, dtype) + u), "shift not exact"
        for causal in (False, True):
            _close(orc.forward(q, ks, v, dtype, 0.05, causal),
                   orc.forward(q, k, v, dtype, 0.05, causal), 1e-12,
                   f"key shift {dtype} causal={causal}")


def check_linearity_in_v(orc):
    """O is linear in V: O(V1 + V2) = O(V1) + O(V2)."""
    for dtype in DTYPES:
        shape = (1, 2, 33, 64)
        q, k = (rand_bits(shape, dtype, s) for s in (101, 102))
        v1 = dyadic_bits(shape, dtype, 103)
        v2 = dyadic_bits(shape, dtype, 104)
        v12 = round_to_storage((np_decode(v1, dtype) + np_decode(v2, dtype)).astype(np.float32), dtype)
        for causal in (False, True):
            lhs = orc.forward(q, k, v12, dtype, 0.125, causal)
            rhs = orc.forward(q, k, v1, dtype, 0.125, causal) + orc.forward(q, k, v2, dtype, 0.125,
                                                                              causal)
            _close(lhs, rhs, 1e-12, f"linearity {dtype} causal={causal}")


def check_causal_prefix(orc):
    """Causal row i equals non-causal attention of query i over keys 0..i."""
    dtype = "bf16"
    shape = (1, 1, 30, 64)
    q, k, v = (rand_bits(shape, dtype, s, 2.0) for s in (111, 112, 113))
    causal = orc.forward(q, k, v, dtype, 0.125, True)[0, 0]
    for i in (0, 1, 2, 7, 15, 29):
        sub = [np.ascontiguousarray(t[:, :, : i + 1]) for t in (q, k, v)]
        full = orc.forward(*sub, dtype, 0.125, False)[0, 0, i]
        _close(causal[i], full, 1e-14, f"causal prefix row {i}")


def check_head_independence(orc):
    """Each (b, h) slice is computed on its own: a batched call equals one
    call per head."""
    dtype = "f16"
    shape = (2, 3, 20, 64)
    q, k, v = (rand_bits(shape, dtype, s) for s in (121, 122, 123))
    for causal in (False, True):
        batched = orc.forward(q, k, v, dtype, 0.125, causal)
        for b in range(2):
            for h in range(3):
                one = orc.forward(*(np.ascontiguousarray(t[b:b + 1, h:h + 1]) for t in (q, k, v)),
                                  dtype, 0.125, causal)
                _close(batched[b:b + 1, h:h + 1], one, 0.0, f"head {b},{h} causal={causal}")


def check_rows_match_forward(orc):
    """The selected-rows entry point returns the same rows as the full pass."""
    dtype = "f16"
    shape = (2, 2, 50, 96)
    q, k, v = (rand_bits(shape, dtype, s) for s in (131, 132, 133))
    rng = np.random.default_rng(134)
    bh = rng.integers(0, 4, size=25)
    ri = rng.integers(0, 50, size=25)
    for causal in (False, True):
        full = orc.forward(q, k, v, dtype, 0.125, causal).reshape(4, 50, 96)
        got = orc.rows(q, k, v, dtype, 0.125, causal, bh, ri)
        _close(got, full[bh, ri], 0.0, f"rows vs forward causal={causal}")


def brute_force_lse(qf, kf, scale, causal):
    """ln sum_j exp(scale * q_i . k_j) over the visible keys, in 40-digit
    decimal arithmetic without the max-subtraction, one (N, D) head."""
    getcontext().prec = 40
    N, D = qf.shape
    sc = Decimal(float(scale))
    out = np.zeros(N)
    for i in range(N):
        tot = Decimal(0)
        for j in range(N):
            if causal and j > i:
                continue
            s = sum((Decimal(float(qf[i, d])) * Decimal(float(kf[j, d])) for d in range(D)),
                    Decimal(0))
            tot += (s * sc).exp()
        out[i] = float(tot.ln())
    return out


def check_lse_brute_force_decimal(orc):
    """The log-sum-exp output on tiny heads against the 40-digit evaluation."""
    cases = [((1, 1, 1, 2), 1.0), ((1, 2, 5, 4), None), ((2, 1, 8, 4), 0.9), ((1, 1, 7, 3), -0.6)]
    seed = 77
    for dtype in DTYPES:
        for causal in (False, True):
            for shape, scale in cases:
                seed += 1
                q = rand_bits(shape, dtype, seed, 1.5)
                k = rand_bits(shape, dtype, seed + 1000, 1.5)
                v = rand_bits(shape, dtype, seed + 2000)
                sc = scale if scale is not None else 1.0 / math.sqrt(shape[3])
                _, lse = orc.forward(q, k, v, dtype, sc, causal, return_lse=True)
                qf, kf = (np_decode(t, dtype) for t in (q, k))
                for b in range(shape[0]):
                    for h in range(shape[1]):
                        ref = brute_force_lse(qf[b, h], kf[b, h], sc, causal)
                        _close(lse[b, h], ref, 1e-13,
                               f"lse brute force {dtype} causal={causal} shape={shape} head={b},{h}")


def check_lse_closed_forms(orc):
    """Log-sum-exp closed forms: one key gives the score itself; identical
    keys give s + ln(visible count); a zero scale gives ln(visible count);
    two keys give max + ln(1 + exp(-|s0 - s1|)); and torch.logsumexp of the
    masked float64 scores (a library routine) on a ragged head."""
    import torch
    for dtype in DTYPES:
        q, k, v = (rand_bits((1, 2, 1, 32), dtype, s) for s in (301, 302, 303))
        _, lse = orc.forward(q, k, v, dtype, 0.3, False, return_lse=True)
        qf, kf = np_decode(q, dtype), np_decode(k, dtype)
        ref = 0.3 * np.einsum("bhnd,bhnd->bhn", qf, kf)
        _close(lse, ref, 1e-14, f"lse one key {dtype}")
    N = 37
    q = rand_bits((1, 1, N, 16), "f16", 311)
    k1 = rand_bits((1, 1, 1, 16), "f16", 312)
    k = np.ascontiguousarray(np.broadcast_to(k1, (1, 1, N, 16)))
    v = rand_bits((1, 1, N, 16), "f16", 313)
    qf, kf = np_decode(q, "f16")[0, 0], np_decode(k1, "f16")[0, 0, 0]
    for causal in (False, True):
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        _, lse = orc.forward(q, k, v, "f16", 0.25, causal, return_lse=True)
        _close(lse[0, 0], 0.25 * qf @ kf + np.log(cnt), 1e-13, f"lse identical keys causal={causal}")
        _, lse0 = orc.forward(q, rand_bits((1, 1, N, 16), "f16", 314), v, "f16", 0.0, causal,
                              return_lse=True)
        _close(lse0[0, 0], np.log(cnt), 1e-14, f"lse zero scale causal={causal}")
    q, k, v = (rand_bits((1, 1, 2, 8), "f32", s, 1.3) for s in (321, 322, 323))
    qf, kf = np_decode(q, "f32")[0, 0], np_decode(k, "f32")[0, 0]
    _, lse = orc.forward(q, k, v, "f32", 0.7, False, return_lse=True)
    for i in range(2):
        s0, s1 = 0.7 * float(qf[i] @ kf[0]), 0.7 * float(qf[i] @ kf[1])
        ref = max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1)))
        _close(lse[0, 0, i], ref, 1e-14, f"lse two keys row {i}")
    shape = (1, 2, 83, 64)
    q, k, v = (rand_bits(shape, "bf16", s, 2.0) for s in (331, 332, 333))
    qt, kt = (torch.from_numpy(np_decode(t, "bf16")) for t in (q, k))
    for causal in (False, True):
        s = 0.125 * torch.matmul(qt, kt.transpose(-1, -2).contiguous())
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(83, 83, dtype=torch.bool), 1), float("-inf"))
        ref = torch.logsumexp(s, dim=-1).numpy()
        _, lse = orc.forward(q, k, v, "bf16", 0.125, causal, return_lse=True)
        _close(lse, ref, 1e-12, f"lse torch.logsumexp causal={causal}")


def check_lse_key_shift_and_rows(orc):
    """Adding one vector u to every key shifts row i's scores, hence its
    log-sum-exp, by scale * q_i . u; the selected-rows entry point returns the
    same log-sum-exp as the full pass."""
    dtype = "f32"
    shape = (1, 1, 40, 16)
    q = dyadic_bits(shape, dtype, 341)
    k = dyadic_bits(shape, dtype, 342)
    u = dyadic_bits((1, 1, 1, 16), dtype, 343)
    v = rand_bits(shape, dtype, 344)
    ks = np.ascontiguousarray((k + u).astype(np.float32))
    for causal in (False, True):
        _, a = orc.forward(q, k, v, dtype, 0.2, causal, return_lse=True)
        _, b = orc.forward(q, ks, v, dtype, 0.2, causal, return_lse=True)
        shift = 0.2 * (np_decode(q, dtype)[0, 0] @ np_decode(u, dtype)[0, 0, 0])
        _close(b[0, 0] - a[0, 0], shift, 1e-12, f"lse key shift causal={causal}")
        bh = np.zeros(10, dtype=np.int64)
        ri = np.arange(0, 40, 4)
        _, lr = orc.rows(q, k, v, dtype, 0.2, causal, bh, ri, return_lse=True)
        _close(lr, a[0, 0, ri], 0.0, f"lse rows vs forward causal={causal}")


CHECKS = [
    check_decode_known_values,
    check_decode_all_16bit_patterns,
    check_brute_force_decimal,
    check_torch_sdpa_fp64,
    check_single_key,
    check_two_keys_logistic,
    check_uniform_scores_mean,
    check_constant_v,
    check_large_scale_argmax,
    check_rowsums_one,
    check_kv_permutation,
    check_q_permutation,
    check_key_shift,
    check_linearity_in_v,
    check_causal_prefix,
    check_head_independence,
    check_rows_match_forward,
    check_lse_brute_force_decimal,
    check_lse_closed_forms,
    check_lse_key_shift_and_rows,
]
