"""Second, independent statement of paged decode for tiny inputs (a pin for the
oracle, not part of it).

Differences from the oracle on purpose: pure Python floats, `math.exp` and
`math.fsum`; every token is reached one by one through the table
(t -> physical block table[t // bs], row t % bs) instead of gathering whole
blocks; the softmax is normalised over the whole context with an explicit
two-pass max/sum; bf16 is decoded with `struct`; FP8 decodes by the
exponent/mantissa formula written out here again.
"""

import math
import struct


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _fp8(code: int) -> float:
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * math.ldexp(m, -9)
    return sign * math.ldexp(8 + m, e - 10)


def _val(x, kind: str) -> float:
    if kind == "f32":
        return float(x)
    if kind == "bf16":
        return _bf16(x)
    return _fp8(x)


def brute_decode(q, kc, vc, tables, lens, scale, bs, q_kind, c_kind, ks=None, vs=None):
    S, H, D = q.shape
    H_kv = kc.shape[1]
    G = H // H_kv
    sc = float(struct.unpack("<f", struct.pack("<f", scale))[0])
    out = [[[0.0] * D for _ in range(H)] for _ in range(S)]
    for i in range(S):
        n = int(lens[i])
        for h in range(H):
            g = h // G
            qv = [_val(q[i, h, d], q_kind) for d in range(D)]
            scores = []
            for t in range(n):
                b = int(tables[i][t // bs])
                r = t % bs
                kscale = float(ks[b, g]) if ks is not None else 1.0
                dot = math.fsum(qv[d] * _val(kc[b, g, r, d], c_kind) * kscale for d in range(D))
                scores.append(dot * sc)
            if n == 0:
                continue
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            z = math.fsum(w)
            for d in range(D):
                acc = []
                for t in range(n):
                    b = int(tables[i][t // bs])
                    r = t % bs
                    vscale = float(vs[b, g]) if vs is not None else 1.0
                    acc.append(w[t] * _val(vc[b, g, r, d], c_kind) * vscale)
                out[i][h][d] = math.fsum(acc) / z
    return out
