"""Fit of the polynomial in av_exp2.h: 2^f on f in [-1/2, 1/2], minimax in
relative error (Remez exchange), degree 3 and 4, rounded to float32.

This is the "Cody-Waite range reduction plus a polynomial" way of computing an
exponential with fused multiply-adds only (W. J. Cody and W. Waite, Software
Manual for the Elementary Functions, 1980: split x = n + f with n an integer
and |f| <= 1/2, so that 2^x = 2^n * 2^f; 2^n is an exponent-field add and 2^f a
short polynomial on a small interval). The coefficients are our own fit.

    python exp2_fit.py        # prints the coefficients and their error
"""
import numpy as np


def remez(deg, iters=30):
    a, b = -0.5, 0.5
    n = deg + 2
    # Chebyshev alternation points as the starting reference
    x = np.cos(np.pi * np.arange(n)[::-1] / (n - 1)) * (b - a) / 2 + (a + b) / 2
    grid = np.linspace(a, b, 200001)
    for _ in range(iters):
        # solve p(x_i) - 2^x_i = (-1)^i E 2^x_i (relative equioscillation)
        A = np.zeros((n, n))
        for i in range(n):
            A[i, :deg + 1] = x[i] ** np.arange(deg + 1)
            A[i, deg + 1] = -((-1) ** i) * 2.0 ** x[i]
        sol = np.linalg.solve(A, 2.0 ** x)
        c = sol[:deg + 1]
        err = (np.polyval(c[::-1], grid) - 2.0 ** grid) / 2.0 ** grid
        # new reference: the extrema of the error, one per sign run
        idx = []
        sign = np.sign(err)
        start = 0
        for k in range(1, len(grid) + 1):
            if k == len(grid) or sign[k] != sign[start]:
                seg = np.arange(start, k)
                idx.append(seg[np.argmax(np.abs(err[seg]))])
                start = k
        if len(idx) < n:
            break
        idx = np.array(idx)
        while len(idx) > n:  # drop the smallest end extremum
            idx = idx[1:] if abs(err[idx[0]]) < abs(err[idx[-1]]) else idx[:-1]
        x = grid[idx]
    c32 = c.astype(np.float32)
    err32 = (np.polyval(c32.astype(np.float64)[::-1], grid) - 2.0 ** grid) / 2.0 ** grid
    return c32, float(np.abs(err32).max())


if __name__ == "__main__":
    for deg in (3, 4):
        c, e = remez(deg)
        print(f"degree {deg}: max relative error {e:.3e}")
        for i, v in enumerate(c):
            print(f"  c{i} = {float(v)!r}f  ({float(v).hex()})")
