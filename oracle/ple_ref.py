"""Oracle of the PLE short convolution and grouped RMSNorm — test infrastructure.

Engram API page ("nemo_automodel.components.models.qwen3_8_flash_next.engram"),
Qwen3_8_FlashNextPLELayer:
  * _causal_short_conv: a causal depthwise convolution over the sequence of a
    [batch, sequence, channels] tensor with "left zero history"; kernel width
    conv_kernel_size (4) and dilation short_conv_dilation = ngram_size (3), so
    the receptive field is 1 + (4 - 1) * 3 = 10 tokens and a context-parallel
    shard needs the preceding nine tokens (the halo);
  * init_weights: the convolution starts at zero.
Layers API page ("nemo_automodel.components.models.qwen3_8_flash_next.layers"),
Qwen3_8_FlashNextGroupedRMSNorm and _grouped_rms_norm_fp32: Gemma-style RMS
normalisation of each group of `group_size` features, computed in fp32, with an
additive scale: the learned weight starts at zero and the output is
x / sqrt(mean(x^2) + eps) * (1 + weight).

Readings where the pages are silent: tap k of the kernel multiplies the input
(K - 1 - k) * dilation positions back (the last tap is the current token, as
a left-padded convolution has it); the bias is optional (zero-start); every
batch row has its own zero history.  All arithmetic here is fp64, in plain
loops over taps and groups.
"""
import numpy as np


def short_conv(x, weight, bias=None, dilation=3, halo=None):
    """x [B, S, C]; weight [C, K]; bias [C] or None; halo [B, (K-1)*dilation, C]
    (the tokens before position 0) or None for zero history.  Returns y [B, S, C]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    B, S, C = x.shape
    K = w.shape[1]
    H = (K - 1) * dilation
    hist = np.zeros((B, H, C)) if halo is None else np.asarray(halo, dtype=np.float64)
    full = np.concatenate([hist, x], axis=1)          # position t of x is H + t here
    y = np.zeros((B, S, C))
    for k in range(K):
        back = (K - 1 - k) * dilation
        y += w[:, k] * full[:, H - back:H - back + S, :]
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)
    return y


def short_conv_backward(x, dy, weight, dilation=3, halo=None):
    """Gradients of short_conv: (dx [B,S,C], dweight [C,K], dbias [C], dhalo [B,H,C])."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    B, S, C = x.shape
    K = w.shape[1]
    H = (K - 1) * dilation
    hist = np.zeros((B, H, C)) if halo is None else np.asarray(halo, dtype=np.float64)
    full = np.concatenate([hist, x], axis=1)
    dfull = np.zeros_like(full)
    dw = np.zeros((C, K))
    for k in range(K):
        back = (K - 1 - k) * dilation
        src = full[:, H - back:H - back + S, :]
        dw[:, k] = (dy * src).sum(axis=(0, 1))
        dfull[:, H - back:H - back + S, :] += w[:, k] * dy
    return dfull[:, H:, :], dw, dy.sum(axis=(0, 1)), dfull[:, :H, :]


def grouped_rms_norm(x, weight, group_size, eps=1e-6):
    """x [..., hidden]; weight [hidden]; each group of group_size features normalised."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    shape = x.shape
    g = x.reshape(-1, shape[-1] // group_size, group_size)
    inv = 1.0 / np.sqrt((g * g).mean(axis=-1, keepdims=True) + eps)
    y = (g * inv).reshape(-1, shape[-1]) * (1.0 + w)
    return y.reshape(shape)


def grouped_rms_norm_backward(x, dy, weight, group_size, eps=1e-6):
    """Gradients of grouped_rms_norm: (dx [..., hidden], dweight [hidden])."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    shape = x.shape
    hidden = shape[-1]
    g = x.reshape(-1, hidden // group_size, group_size)
    inv = 1.0 / np.sqrt((g * g).mean(axis=-1, keepdims=True) + eps)
    n = g * inv
    dn = (dy.reshape(-1, hidden) * (1.0 + w)).reshape(g.shape)
    dx = inv * (dn - n * (dn * n).mean(axis=-1, keepdims=True))
    dw = (dy.reshape(-1, hidden) * n.reshape(-1, hidden)).sum(axis=0)
    return dx.reshape(shape), dw
