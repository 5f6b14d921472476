"""Per-head RMS normalisation, fp64 (oracle; test infrastructure only).

Source: the TensorTonic problem page "Static Arguments in jit" (problem statement,
its normalisation formula, "Examples" and "Constraints"). A token's feature vector
of width D is cut into H heads of width Dh = D/H; head h is features h*Dh .. (h+1)*Dh-1.
Each head vector v becomes v / sqrt(mean_j v_j^2 + eps) with eps = 1e-6 inside the
square root, so an all-zero head stays zero. There is no learned gain.
"""
import numpy as np

RMS_EPS = 1e-6


def rms_rows(x, eps: float = RMS_EPS) -> np.ndarray:
    """Normalise every vector along the last axis: v / sqrt(mean(v^2) + eps), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def per_head_rms_norm(x, num_heads: int, eps: float = RMS_EPS) -> dict:
    """The page's function: x of shape (B, T, D) -> {"heads": (B, H, T, Dh), "merged": (B, T, D)}.

    ``heads[b, h, t]`` is head h of token t of sample b after normalisation; ``merged`` puts
    the normalised heads back in the original feature order.
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, D = x.shape
    if D % num_heads:
        raise ValueError("num_heads must divide the feature width")
    Dh = D // num_heads
    split = x.reshape(B, T, num_heads, Dh)          # [b, t, h, :] is head h of token t
    normed = rms_rows(split, eps)
    heads = np.swapaxes(normed, 1, 2)               # (B, H, T, Dh)
    merged = normed.reshape(B, T, D)                # heads back in feature order
    return {"heads": heads, "merged": merged}
