"""Randomized Walsh-Hadamard rotation, written as an explicit matrix (fp64).

Source: "Closing - The Three-Step Summary", Step 1 (Rotate): each KV vector is
multiplied by a random rotation, in practice a Walsh-Hadamard transform combined
with random signs; the rotation is a change of coordinates that keeps inner
products unchanged. "What the Paper Doesn't Tell You", Finding 4: the WHT needs
only one random sign vector (16 bytes at d=128) and O(d log d) work instead of a
dense d x d matrix. The same finding names the paper's own rotation: a dense random
orthogonal matrix from a QR decomposition (a d x d matrix, O(d^2) work per vector),
kept here as ``qr_rotation`` for the comparison.

Reading adopted (the pages give no formula): R = H_d diag(s) / sqrt(d), with H_d
the Sylvester Hadamard matrix in natural order (H_1 = [1], H_2n = [[H_n, H_n],
[H_n, -H_n]]) and s the +-1 sign vector. R is orthogonal, so R^{-1} = R^T =
diag(s) H_d / sqrt(d). The oracle builds the matrix explicitly (scipy's
``hadamard`` is Sylvester's construction) and multiplies; it never uses a
butterfly.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.linalg import hadamard as _sylvester


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (power of two), fp64 entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    return _sylvester(d).astype(np.float64)


def sign_vector(sign_words, d: int) -> np.ndarray:
    """+-1 vector from packed bits: bit i of word i//32 (LSB first) set -> s_i = -1."""
    w = np.asarray(sign_words, dtype=np.uint32)
    i = np.arange(d)
    bit = (w[i // 32] >> (i % 32).astype(np.uint32)) & np.uint32(1)
    return np.where(bit == 1, -1.0, 1.0)


def rotation_matrix(sign_words, d: int) -> np.ndarray:
    """R = H_d diag(s) / sqrt(d)."""
    s = sign_vector(sign_words, d)
    return hadamard(d) * s[None, :] / math.sqrt(d)


def rotate(u: np.ndarray, sign_words) -> np.ndarray:
    """Rows of u (N, d) mapped to R u."""
    u = np.asarray(u, dtype=np.float64)
    R = rotation_matrix(sign_words, u.shape[-1])
    return u @ R.T


def unrotate(y: np.ndarray, sign_words) -> np.ndarray:
    """Rows of y (N, d) mapped to R^T y (the inverse rotation)."""
    y = np.asarray(y, dtype=np.float64)
    R = rotation_matrix(sign_words, y.shape[-1])
    return y @ R


def qr_rotation(gauss) -> np.ndarray:
    """The dense random rotation: the orthogonal factor Q of the QR decomposition G = Q T of a square iid
    Gaussian matrix G, made unique by the convention diag(T) > 0 (T upper triangular), which makes Q
    Haar-distributed. The pages name the decomposition, not the convention; the rotation is y = Q u. Pins:
    orthogonality, the triangular factor, and classical Gram-Schmidt on a small matrix (tests/pins.py)."""
    G = np.asarray(gauss, dtype=np.float64)
    Q, T = np.linalg.qr(G)
    s = np.where(np.diag(T) < 0, -1.0, 1.0)
    return Q * s[None, :]
