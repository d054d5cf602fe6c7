"""The weightless linear forward, in fp64 on the CPU.

Definition ("Add a new model architecture" page, introduction; "The theta
bundle"): a projection weight is replaced by a shared block W0, a per-row scale
s and a low-rank delta (U, V), and the projection of x is rebuilt as

    y = s * (W0 x) + U (V^T x)                       (factored form)

which is the same linear map as the explicit effective weight that the
precompute-outside path forms once at load time ("Override the graph build",
step 5):

    W_eff = diag(s) W0 + U V^T,     y = W_eff x      (explicit form)

Shapes (row-vector convention, tokens are rows): x [T, K], W0 [N, K], s [N],
U [N, r], V [K, r], y [T, N].  All inputs are the exact stored values (bf16 /
fp32) upcast to fp64; nothing is rounded here.

Stacked calls ("Quality (Gemma 4 31B)" page, "Kernel optimizations > GEMM
path"): q/k/v (and gate/up) of one layer share x; the stacked result is the
per-child results concatenated along N in the order q, k, v / gate, up.  With
K=V tying on a layer type ("Decompose HF weights: the mixed-attention case"),
v has no bundle and its output is k's output.
"""
import math

import numpy as np

# MLP hidden activations by name ("Quality (Gemma 4 31B)" page, "Activation
# function fix": Gemma 3 and 4 use gelu with the tanh approximation, and a
# hardcoded silu broke the model; "Add a new model architecture" page, "Route
# the MLP through config.hidden_activation": the activation is a parameter of
# the model, never fixed in the layer).  Each is written from its definition.
ACTIVATIONS = ("gelu_tanh", "silu", "gelu")


def activation(name, x):
    """gelu_tanh: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)));
    silu: x / (1 + e^-x);  gelu: x Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    x = np.asarray(x, np.float64)
    if name == "gelu_tanh":
        return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))
    if name == "silu":
        return x / (1.0 + np.exp(-x))
    if name == "gelu":
        return 0.5 * x * (1.0 + np.vectorize(math.erf, otypes=[np.float64])(x / math.sqrt(2.0)))
    raise ValueError(f"unknown activation {name!r}")


def dense(x, W):
    """y = x W^T: the plain dense projection."""
    return np.asarray(x, np.float64) @ np.asarray(W, np.float64).T


def factored(x, W0, s, U, V):
    """y = (x W0^T) * s + (x V) U^T, evaluated in that order in fp64."""
    x = np.asarray(x, np.float64)
    p = x @ np.asarray(W0, np.float64).T                 # shared-block product [T, N]
    y = p * np.asarray(s, np.float64)[None, :]           # per-row scale
    r = np.asarray(U).shape[1]
    if r:
        z = x @ np.asarray(V, np.float64)                # thin reduction V^T x  [T, r]
        y = y + z @ np.asarray(U, np.float64).T          # low-rank delta        [T, N]
    return y


def effective_weight(W0, s, U, V):
    """W_eff = diag(s) W0 + U V^T."""
    W = np.asarray(s, np.float64)[:, None] * np.asarray(W0, np.float64)
    if np.asarray(U).shape[1]:
        W = W + np.asarray(U, np.float64) @ np.asarray(V, np.float64).T
    return W


def explicit(x, W0, s, U, V):
    """y = x W_eff^T with the effective weight formed first."""
    return dense(x, effective_weight(W0, s, U, V))


def stacked(x, children):
    """Concatenate child results along N.  ``children`` is a list of
    (W0, s, U, V) tuples, or the string "dup" for a child whose output is the
    previous child's output (K=V tying)."""
    outs = []
    for ch in children:
        if isinstance(ch, str) and ch == "dup":
            outs.append(outs[-1].copy())
        else:
            outs.append(factored(x, *ch))
    return np.concatenate(outs, axis=1)


def gate_up_act(x, gate, up, name):
    """The MLP's gated hidden state h = act(gate x) * (up x), with gate and up
    each a (W0, s, U, V) bundle evaluated in the factored form."""
    return activation(name, factored(x, *gate)) * factored(x, *up)
