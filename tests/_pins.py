"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes an ``oracle.Oracle`` and returns a list of failure messages
(empty when the pin holds), so the same pins can be run against the real
oracle and against deliberately broken copies of it (mutation tests).

What pins what:

* ``half_decode``       fp16 -> fp64 against numpy's conversion, all 65536 patterns
* ``pack_golden``       hand-derived packed words (tests/golden/pack_examples.txt)
* ``single_code``       every code value at every position sets exactly its bits
* ``round_trip``        unpack(pack(Q)) == Q and pack(unpack(W)) == W
* ``forward_golden``    hand-computed products (tests/golden/forward_examples.txt)
* ``integer_matmul``    s = 1, b = 0, integer x: exact numpy int64 Q @ X^T
* ``dyadic_exhaustive`` all 16^4 codes of a 4-code window, dyadic s/b/x: exact
                        integer evaluation of the definition, and the factored form
* ``one_hot``           x = e_k gives s[n,k/G] q[n,k] + b[n,k/G] (numpy, from the codes)
* ``ones``              x = 1 gives sum_g (s_g sum q + G b_g)
* ``zero_codes``        q = 0 gives sum_g b_g XS_g
* ``linearity``         y(x1 + x2) = y(x1) + y(x2)
* ``row_invariance``    each row of an M-row result equals the 1-row result bitwise;
                        selected-row and multi-thread evaluation are bitwise equal
* ``absum``             A = |y| when every term is non-negative, A >= |y| always
"""
from __future__ import annotations

from pathlib import Path

import numpy as np

GOLDEN = Path(__file__).resolve().parent / "golden"


def _h(values) -> np.ndarray:
    return np.asarray(values, dtype=np.float64).astype(np.float16)


def _codes_to_words_numpy(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack with numpy's bit routines (LSB-first), independent of the oracle's loops."""
    N, K = codes.shape
    # bit j of code k -> stream bit k*bits + j
    b = ((codes[:, :, None].astype(np.uint32) >> np.arange(bits, dtype=np.uint32)) & 1).astype(np.uint8)
    stream = b.reshape(N, K * bits)
    packed_bytes = np.packbits(stream, axis=1, bitorder="little")
    return packed_bytes.view("<u4").reshape(N, K * bits // 32)


# --------------------------------------------------------------------------
def bf16_decode(o) -> list[str]:
    """Every bfloat16 pattern against numpy's float32 decode of the same bits
    in the upper half of a binary32."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = o.bf16_to_double(pats)
    with np.errstate(invalid="ignore"):  # signalling NaN patterns
        want = (pats.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(want)
    bad = ~((got == want) | (nan & np.isnan(got)))
    bad |= (want == 0) & (np.signbit(got) != np.signbit(want))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        return [f"bf16 0x{int(pats[i]):04x}: oracle {got[i]!r}, numpy {want[i]!r} ({int(bad.sum())} bad)"]
    return []


def _bf16_bits_exact(values) -> np.ndarray:
    """Bit patterns of values that bfloat16 holds exactly (asserted)."""
    f = np.asarray(values, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f), "value not exact in bf16"
    return bits


def bf16_operands(o) -> list[str]:
    """Values exact in both fp16 and bf16 (dyadic, few significant bits, in
    range) give the same product whether x, s and b are passed as fp16 or as
    bf16: the bf16 path decodes every operand, and each in its own place."""
    fails = []
    rng = np.random.default_rng(77)
    for bits, G, K in ((4, 32, 128), (5, 64, 192), (8, 32, 96)):
        M, N = 3, 5
        x = rng.integers(-64, 65, size=(M, K)) / 8.0                 # k/8, |x| <= 8
        s = rng.integers(1, 17, size=(N, K // G)) * 2.0 ** -9         # j * 2^-9
        b = rng.integers(-16, 17, size=(N, K // G)) * 2.0 ** -7       # i * 2^-7
        words = rng.integers(0, 1 << 32, size=(N, K * bits // 32), dtype=np.uint32)
        y16, a16 = o.forward(_h(x), words, _h(s), _h(b), bits, G)
        yb, ab = o.forward(_bf16_bits_exact(x), words, _bf16_bits_exact(s), _bf16_bits_exact(b),
                           bits, G, dtype="bf16")
        if not (np.array_equal(y16, yb) and np.array_equal(a16, ab)):
            fails.append(f"bits={bits} G={G}: bf16 and fp16 operands of equal value disagree")
        rows = np.array([4, 0, 2])
        yr, _ = o.forward_rows(_bf16_bits_exact(x), words, _bf16_bits_exact(s), _bf16_bits_exact(b),
                               bits, G, rows, dtype="bf16")
        if not np.array_equal(yr, y16[:, rows]):
            fails.append(f"bits={bits} G={G}: bf16 row list disagrees")
    return fails


def half_decode(o) -> list[str]:
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = o.half_to_double(pats)
    want = pats.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    bad = ~((got == want) | (nan & np.isnan(got)))
    # signed zeros must keep their sign
    bad |= (want == 0) & (np.signbit(got) != np.signbit(want))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        return [f"half 0x{int(pats[i]):04x}: oracle {got[i]!r}, numpy {want[i]!r} ({int(bad.sum())} bad)"]
    return []


def _parse_pack_golden():
    for line in (GOLDEN / "pack_examples.txt").read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        head, assigns, words = (p.strip() for p in line.split("|"))
        bits, K = (int(v) for v in head.split())
        codes = np.zeros((1, K), dtype=np.uint8)
        for a in assigns.split():
            k, v = a.split("=")
            codes[0, int(k)] = int(v, 0)
        expect = np.array([int(w, 16) for w in words.split()], dtype=np.uint32)[None, :]
        yield bits, K, codes, expect


def pack_golden(o) -> list[str]:
    fails = []
    for bits, K, codes, expect in _parse_pack_golden():
        got = o.pack(codes, bits)
        if got.shape != expect.shape or not np.array_equal(got, expect):
            fails.append(f"pack bits={bits} K={K}: got {[hex(int(v)) for v in got.ravel()]}, "
                         f"want {[hex(int(v)) for v in expect.ravel()]}")
        back = o.unpack(expect, K, bits)
        if not np.array_equal(back, codes):
            fails.append(f"unpack bits={bits} K={K} of golden words differs from the codes")
    return fails


def single_code(o) -> list[str]:
    fails = []
    for bits in (2, 3, 4, 5, 6, 8):
        K = 64  # two groups of 32
        values = np.arange(1, 1 << bits, dtype=np.uint32)
        rows = []
        for k in range(K):
            for v in values:
                rows.append((k, int(v)))
        codes = np.zeros((len(rows), K), dtype=np.uint8)
        for r, (k, v) in enumerate(rows):
            codes[r, k] = v
        words = o.pack(codes, bits)
        # expected: bit (k*bits + j) set iff bit j of v is set, nothing else
        expect = np.zeros_like(words)
        for r, (k, v) in enumerate(rows):
            for j in range(bits):
                if (v >> j) & 1:
                    t = k * bits + j
                    expect[r, t // 32] |= np.uint32(1 << (t % 32))
        if not np.array_equal(words, expect):
            r = int(np.flatnonzero((words != expect).any(axis=1))[0])
            fails.append(f"single code bits={bits} (k, v)={rows[r]}: words {words[r]} != {expect[r]}")
        if not np.array_equal(o.unpack(expect, K, bits), codes):
            fails.append(f"single code unpack bits={bits}")
    return fails


def round_trip(o) -> list[str]:
    fails = []
    rng = np.random.default_rng(1234)
    for bits in (2, 3, 4, 5, 6, 8):
        for K in (32, 64, 96, 512):
            Q = rng.integers(0, 1 << bits, size=(7, K), dtype=np.uint8)
            W = o.pack(Q, bits)
            if not np.array_equal(W, _codes_to_words_numpy(Q, bits)):
                fails.append(f"pack vs numpy packbits bits={bits} K={K}")
            if not np.array_equal(o.unpack(W, K, bits), Q):
                fails.append(f"unpack(pack(Q)) != Q bits={bits} K={K}")
            Wr = rng.integers(0, 1 << 32, size=(5, K * bits // 32), dtype=np.uint32)
            if not np.array_equal(o.pack(o.unpack(Wr, K, bits), bits), Wr):
                fails.append(f"pack(unpack(W)) != W bits={bits} K={K}")
    return fails


def _x_rule(rule: str, K: int) -> np.ndarray:
    k = np.arange(K)
    if rule == "ones":
        return np.ones(K)
    if rule == "alt":
        return np.where(k % 2 == 0, 1.0, -1.0)
    if rule == "1,2":
        return np.where(k < K // 2, 1.0, 2.0)
    raise ValueError(rule)


def _codes_rule(rule: str, K: int) -> np.ndarray:
    k = np.arange(K)
    if rule == "k%16":
        return k % 16
    if "," in rule:
        a, b = (int(v) for v in rule.split(","))
        return np.where(k % 2 == 0, a, b)
    return np.full(K, int(rule))


def forward_golden(o) -> list[str]:
    fails = []
    for line in (GOLDEN / "forward_examples.txt").read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        name, shape, crule, sc, bi, xrule, y_s, a_s = (p.strip() for p in line.split("|"))
        bits, K, G = (int(v) for v in shape.split())
        codes = _codes_rule(crule, K).astype(np.uint8)[None, :]
        words = _codes_to_words_numpy(codes, bits)
        s = _h([float(v) for v in sc.split()])[None, :]
        b = _h([float(v) for v in bi.split()])[None, :]
        x = _h(_x_rule(xrule, K))[None, :]
        y, a = o.forward(x, words, s, b, bits, G, nthreads=1)
        yf = o.forward_factored(x, words, s, b, bits, G, nthreads=1)
        if y[0, 0] != float(y_s) or a[0, 0] != float(a_s) or yf[0, 0] != float(y_s):
            fails.append(f"golden {name}: y={y[0, 0]} A={a[0, 0]} factored={yf[0, 0]}, "
                         f"want y={y_s} A={a_s}")
    return fails


def integer_matmul(o) -> list[str]:
    fails = []
    rng = np.random.default_rng(99)
    for bits in (2, 3, 4, 5, 6, 8):
        for G in (32, 64):
            M, K, N = 3, 128, 37
            Q = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
            X = rng.integers(-8, 9, size=(M, K))
            words = _codes_to_words_numpy(Q, bits)
            s = np.ones((N, K // G), dtype=np.float16)
            b = np.zeros((N, K // G), dtype=np.float16)
            y, _ = o.forward(X.astype(np.float16), words, s, b, bits, G, nthreads=2)
            want = X.astype(np.int64) @ Q.astype(np.int64).T
            if not np.array_equal(y, want.astype(np.float64)):
                fails.append(f"integer matmul bits={bits} G={G}: max |diff| {np.abs(y - want).max()}")
    return fails


def dyadic_exhaustive(o) -> list[str]:
    """All 16^4 code combinations in a 4-code window of an 8-code row (4-bit, G = 2).

    s = S * 2^-6, b = B * 2^-6, x = X * 2^-2 with small integers, so
    y * 2^8 = sum_k (S q + B) X is an integer that int64 evaluates exactly;
    both oracle forms must hit it exactly.
    """
    bits, K, G = 4, 8, 2
    grid = np.stack(np.meshgrid(*[np.arange(16)] * 4, indexing="ij"), axis=-1).reshape(-1, 4)
    N = grid.shape[0]
    Q = np.empty((N, K), dtype=np.uint8)
    Q[:, :4] = grid
    Q[:, 4:] = np.array([3, 9, 14, 6], dtype=np.uint8)
    S = np.array([5, -3, 7, 2])       # per group (K/G = 4 groups)
    B = np.array([-6, 11, 1, -13])
    X = np.array([[4, -2, 1, 8, -5, 3, -7, 2],
                  [-1, 6, -3, -4, 2, 5, 1, -8]])
    s = _h(np.tile(S * 2.0 ** -6, (N, 1)))
    b = _h(np.tile(B * 2.0 ** -6, (N, 1)))
    x = _h(X * 2.0 ** -2)
    words = _codes_to_words_numpy(Q, bits)
    Wint = S[np.arange(K) // G][None, :] * Q.astype(np.int64) + B[np.arange(K) // G][None, :]
    want = (X.astype(np.int64) @ Wint.T).astype(np.float64) * 2.0 ** -8
    y, a = o.forward(x, words, s, b, bits, G)
    yf = o.forward_factored(x, words, s, b, bits, G)
    fails = []
    if not np.array_equal(y, want):
        fails.append(f"dyadic dequant-then-dot != exact integer value ({int((y != want).sum())} elements)")
    if not np.array_equal(yf, want):
        fails.append(f"dyadic factored form != exact integer value ({int((yf != want).sum())} elements)")
    awant = (np.abs(X.astype(np.int64))[:, None, :] * np.abs(Wint)[None, :, :]).sum(-1) * 2.0 ** -8
    if not np.array_equal(a, awant):
        fails.append("dyadic A != exact sum |w x|")
    return fails


def _random_problem(rng, M, K, N, bits, G):
    Q = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    s = _h(rng.uniform(0.005, 0.02, size=(N, K // G)))
    b = _h(rng.uniform(-0.1, 0.1, size=(N, K // G)))
    x = _h(rng.standard_normal((M, K)))
    return Q, _codes_to_words_numpy(Q, bits), s, b, x


def one_hot(o) -> list[str]:
    fails = []
    rng = np.random.default_rng(7)
    for bits, G in ((2, 32), (3, 64), (4, 32), (5, 64), (6, 32), (8, 64)):
        K, N = 128, 19
        Q, words, s, b, _ = _random_problem(rng, 1, K, N, bits, G)
        x = np.zeros((K, K), dtype=np.float16)
        x[np.arange(K), np.arange(K)] = 1.0
        y, _ = o.forward(x, words, s, b, bits, G)
        g = np.arange(K) // G
        want = (s.astype(np.float64)[:, g] * Q + b.astype(np.float64)[:, g]).T  # [k, n]
        if not np.array_equal(y, want):
            fails.append(f"one-hot bits={bits} G={G}: {int((y != want).sum())} mismatches")
    return fails


def ones(o) -> list[str]:
    fails = []
    rng = np.random.default_rng(8)
    for bits, G in ((2, 64), (3, 32), (4, 32), (5, 32), (6, 64), (8, 32)):
        K, N = 256, 23
        Q, words, s, b, _ = _random_problem(rng, 1, K, N, bits, G)
        x = np.ones((1, K), dtype=np.float16)
        y, a = o.forward(x, words, s, b, bits, G)
        qsum = Q.reshape(N, K // G, G).astype(np.float64).sum(-1)
        want = (s.astype(np.float64) * qsum + G * b.astype(np.float64)).sum(-1)
        if not np.allclose(y[0], want, rtol=0, atol=1e-12 * a[0].max()):
            fails.append(f"x=1 bits={bits} G={G}: max |diff| {np.abs(y[0] - want).max()}")
    return fails


def zero_codes(o) -> list[str]:
    fails = []
    rng = np.random.default_rng(9)
    for bits, G in ((4, 32), (6, 64)):
        M, K, N = 2, 192, 11
        _, _, s, b, x = _random_problem(rng, M, K, N, bits, G)
        words = np.zeros((N, K * bits // 32), dtype=np.uint32)
        y, a = o.forward(x, words, s, b, bits, G)
        xs = x.astype(np.float64).reshape(M, K // G, G).sum(-1)
        want = xs @ b.astype(np.float64).T
        if not np.allclose(y, want, rtol=0, atol=1e-12 * a.max()):
            fails.append(f"zero codes bits={bits} G={G}: max |diff| {np.abs(y - want).max()}")
    return fails


def linearity(o) -> list[str]:
    fails = []
    rng = np.random.default_rng(10)
    bits, G, K, N = 5, 32, 160, 13
    Q, words, s, b, _ = _random_problem(rng, 1, K, N, bits, G)
    # small dyadic values so x1 + x2 is exact in fp16
    x1 = _h(rng.integers(-64, 65, size=(1, K)) / 64.0)
    x2 = _h(rng.integers(-64, 65, size=(1, K)) / 64.0)
    y1, a1 = o.forward(x1, words, s, b, bits, G)
    y2, a2 = o.forward(x2, words, s, b, bits, G)
    y12, _ = o.forward(_h(x1.astype(np.float64) + x2.astype(np.float64)), words, s, b, bits, G)
    if not np.allclose(y12, y1 + y2, rtol=0, atol=1e-12 * (a1 + a2).max()):
        fails.append(f"linearity: max |diff| {np.abs(y12 - y1 - y2).max()}")
    return fails


def row_invariance(o) -> list[str]:
    fails = []
    rng = np.random.default_rng(11)
    bits, G, M, K, N = 4, 32, 5, 256, 29
    _, words, s, b, x = _random_problem(rng, M, K, N, bits, G)
    y, a = o.forward(x, words, s, b, bits, G, nthreads=3)
    for m in range(M):
        y1, a1 = o.forward(x[m:m + 1], words, s, b, bits, G, nthreads=1)
        if not (np.array_equal(y[m], y1[0]) and np.array_equal(a[m], a1[0])):
            fails.append(f"row {m} of the {M}-row result differs from the 1-row result")
    rows = np.array([28, 0, 7, 7, 13])
    yr, ar = o.forward_rows(x, words, s, b, bits, G, rows, nthreads=2)
    if not (np.array_equal(yr, y[:, rows]) and np.array_equal(ar, a[:, rows])):
        fails.append("selected-row evaluation differs from the full evaluation")
    return fails


def absum(o) -> list[str]:
    fails = []
    rng = np.random.default_rng(12)
    bits, G, M, K, N = 6, 64, 2, 128, 9
    _, words, s, b, x = _random_problem(rng, M, K, N, bits, G)
    y, a = o.forward(x, words, s, b, bits, G)
    if not (a >= np.abs(y)).all():
        fails.append("A < |y| somewhere")
    # all terms non-negative: positive scales, zero biases, non-negative x
    xp = _h(np.abs(x.astype(np.float64)))
    bz = np.zeros_like(b)
    yp, ap = o.forward(xp, words, s, bz, bits, G)
    if not np.allclose(ap, yp, rtol=1e-15, atol=0):
        fails.append("A != y when every term is non-negative")
    return fails


def tiled_layout(o) -> list[str]:
    """The tiled re-layout, checked against word-level closed forms that follow
    from its definition for each supported width at G = 32: lane block c of a
    group is word c of the group's 4 words (4-bit), words 2c, 2c+1 of its 8
    (8-bit), the 16-bit half c of its 2 words (2-bit); a lane's 16-byte unit
    holds consecutive groups; rows past N are zero; (s, b) words are the
    scales and biases of 4 consecutive groups per row, rows of a tile in order."""
    fails = []
    rng = np.random.default_rng(21)
    N, K, G = 37, 512, 32
    for bits in (2, 4, 8):
        W = K * bits // 32
        words = rng.integers(0, 1 << 32, size=(N, W), dtype=np.uint32)
        s = rng.random((N, K // G)).astype(np.float16)
        b = (rng.random((N, K // G)) - 0.5).astype(np.float16)
        tw, tsb = o.repack_tiled(words, s, b, K, bits, G)
        UB = K * bits // 512
        tiles = (N + 15) // 16
        units = tw.view(np.uint32).reshape(tiles, UB, 4, 16, 4)  # [t][u][c][i][dword]
        padded = np.zeros((tiles * 16, W), dtype=np.uint32)
        padded[:N] = words
        rows = padded.reshape(tiles, 16, W)  # [t][i][word]
        wpg = G * bits // 32  # words per group
        if bits == 4:    # unit u: groups 4u..4u+3, word c of each
            want = rows.reshape(tiles, 16, UB, 4, 4)[:, :, :, :, :]  # [t][i][u][group in unit][word c]
            want = want.transpose(0, 2, 4, 1, 3)                    # [t][u][c][i][group in unit]
        elif bits == 8:  # unit u: groups 2u, 2u+1, words 2c, 2c+1 of each
            g8 = rows.reshape(tiles, 16, UB, 2, 4, 2)                # [t][i][u][group][c][half]
            want = g8.transpose(0, 2, 4, 1, 3, 5).reshape(tiles, UB, 4, 16, 4)
        else:            # bits 2: unit u: groups 8u..8u+7, 16-bit half c of each group's 2 words
            halves = rows.reshape(tiles, 16, UB, 8, wpg).view(np.uint16).reshape(tiles, 16, UB, 8, 4)
            want = halves.transpose(0, 2, 4, 1, 3).copy().view(np.uint32)  # pairs of halves -> dwords
        if not np.array_equal(units, want):
            fails.append(f"tiled codes bits={bits}: {int((units != want).sum())} words differ")
        sbw = tsb.reshape(tiles, K // G // 4, 16, 4)            # [t][q][i][e]
        sp = np.zeros((tiles * 16, K // G), dtype=np.uint32)
        sp[:N] = s.view(np.uint16).astype(np.uint32) | (b.view(np.uint16).astype(np.uint32) << 16)
        want_sb = sp.reshape(tiles, 16, K // G // 4, 4).transpose(0, 2, 1, 3)
        if not np.array_equal(sbw, want_sb):
            fails.append(f"tiled (s, b) words bits={bits}: {int((sbw != want_sb).sum())} differ")
    return fails


ALL_PINS = (half_decode, pack_golden, single_code, round_trip, forward_golden,
            integer_matmul, dyadic_exhaustive, one_hot, ones, zero_codes,
            linearity, row_invariance, absum, tiled_layout, bf16_decode, bf16_operands)


def run_all(o) -> dict[str, list[str]]:
    out = {}
    for pin in ALL_PINS:
        try:
            out[pin.__name__] = pin(o)
        except Exception as exc:  # a broken oracle may raise instead of returning wrong values
            out[pin.__name__] = [f"raised {type(exc).__name__}: {exc}"]
    return out
