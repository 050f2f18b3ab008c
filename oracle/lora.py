"""LoRA linear over a frozen base weight (oracle; test infrastructure).

What the pages fix: only the LoRA adapters train; the base stays frozen and is
never given a gradient, and the backward needs the base weight to push the
gradient to the input (dL/dx = W^T dL/dy) (LS-docs "How it works"; About).
Plain LoRA only, no DoRA / VeRA and friends (LS-docs "Honest scope").  Adapter
tensor names lora_A / lora_B follow PEFT (LS-docs "Read this first": the key
names of a saved adapter).

Reading of PEFT's plain LoRA (the pages print none of it): A is [r, K], B is [N, r],
scale s = alpha / r, dropout 0, so for X [M, K] and base W [N, K]

    U  = X A^T                       [M, r]
    Y  = X W^T + s U B^T (+ bias)    [M, N]

and for an upstream gradient dY [M, N]

    G  = dY B                        [M, r]
    dX = dY W + s G A                [M, K]
    dA = s G^T X                     [r, K]
    dB = s dY^T U                    [N, r]

No gradient for W or the bias.  All arrays are float64.
"""
import numpy as np


def linear_fwd(X, W, A, B, s, bias=None):
    U = X @ A.T
    Y = X @ W.T + s * (U @ B.T)
    if bias is not None:
        Y = Y + bias
    return Y, U


def linear_bwd(X, W, A, B, s, dY):
    G = dY @ B
    dX = dY @ W + s * (G @ A)
    dA = s * (G.T @ X)
    dB = s * (dY.T @ (X @ A.T))
    return dX, dA, dB
