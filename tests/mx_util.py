"""MXFP8 matrices in the library's byte layout (codes, then scale planes), built from and read
back into numpy for the tests.  The expected bytes come from the oracle's quantiser; nothing here
quantises or computes the block."""

import numpy as np

import oracle


def _round_up(v, a):
    return (v + a - 1) // a * a


def layout(rows, k):
    """(byte offset of the scale planes, plane stride, total bytes) of a rows x k matrix."""
    po = _round_up(rows * k, 256)
    ps = _round_up(rows, 16)
    return po, ps, po + _round_up((k // 32) * ps, 256)


def encode(vals, x):
    """The oracle's MXFP8 values ``vals`` [rows, k] and scale exponents ``x`` [rows, k / 32] as
    the library's bytes."""
    rows, k = vals.shape
    po, ps, total = layout(rows, k)
    buf = np.zeros(total, np.uint8)
    scale = np.exp2(np.repeat(x.astype(np.float64), 32, axis=1))
    buf[:rows * k] = oracle.e4m3_bits(vals / scale).reshape(-1)
    planes = np.zeros((k // 32, ps), np.uint8)
    planes[:, :rows] = (x + 127).astype(np.uint8).T
    buf[po:po + planes.size] = planes.reshape(-1)
    return buf


def decode(buf, rows, k):
    """Bytes of an MXFP8 matrix -> (codes uint8 [rows, k], scale bytes [rows, k / 32], values)."""
    import torch
    po, ps, _ = layout(rows, k)
    codes = np.asarray(buf[:rows * k], np.uint8).reshape(rows, k)
    sbytes = np.asarray(buf[po:po + (k // 32) * ps], np.uint8).reshape(k // 32, ps)[:, :rows].T
    e4m3 = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vals = e4m3 * np.exp2(np.repeat(sbytes.astype(np.float64) - 127, 32, axis=1))
    return codes, np.ascontiguousarray(sbytes), vals


def oracle_bytes(a):
    """(bytes, values) of the oracle's MXFP8 form of ``a`` [rows, k]."""
    vals, x = oracle.mx_quantize(a)
    return encode(vals, x), vals
