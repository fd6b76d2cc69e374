"""Independent dense numpy routines used to pin the oracle.

Nothing here calls the oracle: the int4 container is decoded with numpy's int8
arithmetic shift and numpy's float16 view, and the products are library matmuls.
They are slow-path special cases (materialise W, multiply densely) that the
oracle's streaming definition must reduce to.
"""
import numpy as np

GS = 64


def decode_nibbles(nib: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """[rows][cols] int8 from packed bytes: low four bits = even column."""
    b = np.asarray(nib, dtype=np.uint8).reshape(rows, cols // 2)
    lo = ((b << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.int8)   # sign-extend bits 0-3
    hi = (b.view(np.int8) >> 4).astype(np.int8)                            # sign-extend bits 4-7
    q = np.empty((rows, cols), dtype=np.int8)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    return q


def decode_scales(sc: np.ndarray, rows: int, cols: int) -> np.ndarray:
    return np.frombuffer(np.ascontiguousarray(sc, dtype=np.uint8).tobytes(), dtype="<f2").astype(
        np.float64).reshape(rows, cols // GS)


def dense_matrix(nib, sc, rows: int, cols: int) -> np.ndarray:
    q = decode_nibbles(nib, rows, cols).astype(np.float64)
    s = np.repeat(decode_scales(sc, rows, cols), GS, axis=1)
    return q * s


def sections(blob: np.ndarray, d: int, f: int):
    w = d * f
    nb, ns = w // 2, (w // GS) * 2
    o = 0
    out = []
    for _ in range(3):
        out.append((blob[o:o + nb], blob[o + nb:o + nb + ns]))
        o += nb + ns
    return out


def dense_expert(blob: np.ndarray, d: int, f: int):
    (gn, gs), (un, us), (dn, ds) = sections(np.asarray(blob, dtype=np.uint8), d, f)
    return dense_matrix(gn, gs, f, d), dense_matrix(un, us, f, d), dense_matrix(dn, ds, d, f)


# int8 container: one two's-complement byte per weight (numpy's int8 view)
def dense_matrix_i8(q8, sc, rows: int, cols: int) -> np.ndarray:
    q = np.asarray(q8, dtype=np.uint8).view(np.int8).reshape(rows, cols).astype(np.float64)
    return q * np.repeat(decode_scales(sc, rows, cols), GS, axis=1)


def dense_expert_i8(blob: np.ndarray, d: int, f: int):
    w = d * f
    ns = (w // GS) * 2
    b = np.asarray(blob, dtype=np.uint8)
    mats, o = [], 0
    for rows, cols in ((f, d), (f, d), (d, f)):
        mats.append(dense_matrix_i8(b[o:o + w], b[o + w:o + w + ns], rows, cols))
        o += w + ns
    return mats


def silu(z):
    from scipy.special import expit
    return z * expit(z)


def dense_ffn(Wg, Wu, Wd, x):
    return Wd @ (silu(Wg @ x) * (Wu @ x))


def dense_moe_all(blobs, shared, R, bias, x, d, f, k):
    """Brute force: every expert evaluated densely, a top-k mask from a stable
    library sort, softmax over the kept logits (scipy)."""
    from scipy.special import softmax
    x = np.asarray(x, dtype=np.float64)
    l = R.astype(np.float64) @ x
    if bias is not None:
        l = l + bias.astype(np.float64)
    E = R.shape[0]
    order = np.lexsort((np.arange(E), -l))
    sel = order[:k]
    w = softmax(l[sel])
    ys = np.stack([dense_ffn(*dense_expert(blobs[e], d, f), x) for e in range(E)])
    mask = np.zeros(E)
    mask[sel] = w
    out = x + mask @ ys
    if shared is not None:
        out = out + dense_ffn(*dense_expert(shared, d, f), x)
    return out, sel, w
