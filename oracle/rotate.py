"""Hadamard rotation of 256-dim rows before key quantisation (test
infrastructure: the CPU oracle; nothing in the product imports it).

[VULKAN] section "沒踩到的坑：注意力旋轉": the attention rotation (a Hadamard
rotation on the attention path) is there to raise the precision of a
quantised KV cache, and the author keeps it on with q8_0 / q5_1 / q4_0 caches.
The pages do not spell the transform out. Reading taken here: the rotation is
the orthonormal Sylvester-Hadamard matrix H_256 / 16 applied to each 256-dim
key row before Q8_0 quantisation and to each query row before attention, so
q . k = (H q / 16) . (H k / 16) exactly in real arithmetic and the attention
is unchanged apart from quantisation error. Values may be rotated too, the
output then rotated once more (H / 16 is its own inverse).

For the quantised bytes to be reproducible bit for bit the binary32
arithmetic is fixed: the fast Walsh-Hadamard butterflies with half-widths
h = 1, 2, 4, ..., 128 in that order, each pair (i, i + h) with bit h of i
clear becoming (x[i] + x[i+h], x[i] - x[i+h]) rounded to binary32, then a
multiplication by 1/16 (exact). With h ascending the butterflies compute
the Sylvester-ordered H_256 (the one scipy.linalg.hadamard builds).
"""
import numpy as np

DIM = 256


def hadamard_matrix(n=DIM):
    """Sylvester-ordered H_n (entries +-1): H_1 = [1], H_2k = [[H, H], [H, -H]]."""
    h = np.ones((1, 1), np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_rows_f64(x):
    """The definition in binary64: rows of x (last axis 256) times H_256^T / 16."""
    x = np.asarray(x, np.float64)
    return x @ hadamard_matrix(x.shape[-1]).T / np.sqrt(x.shape[-1])


def rotate_rows_f32(x):
    """The binary32 butterfly order fixed above. x float32 [..., 256]."""
    y = np.array(x, np.float32, copy=True)
    if y.shape[-1] != DIM:
        raise ValueError("rows must have 256 elements")
    shape = y.shape
    y = y.reshape(-1, DIM)
    h = 1
    while h < DIM:
        v = y.reshape(-1, DIM // (2 * h), 2, h)     # pairs (i, i + h) inside blocks of 2h
        a = v[:, :, 0, :].copy()
        b = v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b                       # binary32 add, rounded
        v[:, :, 1, :] = a - b
        y = v.reshape(-1, DIM)
        h *= 2
    y = y * np.float32(1.0 / 16.0)                  # exact: a power of two
    return y.reshape(shape)
