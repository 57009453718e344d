"""Seeded synthetic Q/K/V for one attention layer of a video diffusion transformer.

This module only produces inputs. It holds none of the clustered-attention
arithmetic, so both the CPU oracle (``oracle/``) and the HIP library may be fed
from it without sharing any of the method's code.

Recipe (the AdaCluster paper measures real DiT activations of CogVideoX-2B,
Wan-2.1 and HunyuanVideo, section 4.1 "Setup"; neither weights nor prompts are
available, so these fields stand in for them):

  tokens are indexed row-major over a (T, Hg, W) latent grid; for every tensor
  X in {Q, K, V} (independent sub-streams), every head h and each of 8 fields f:
      a_f ~ U(0.5, 1.5), u_f ~ N(0, I_D), (kt, ky, kx) ~ U(0, 2), phi_f ~ U(0, 2 pi)
      X[h, (t,y,x)] = sum_f a_f sin(2 pi (kt t/T + ky y/Hg + kx x/W) + phi_f) u_f
                      + 0.1 eps
  eps ~ N(0, 1), or Student-t(3) for the heavy-tailed (HunyuanVideo-shaped) case;
  an optional per-head scale s_h ~ U(0.5, 2) shared by Q, K and V
  (Wan-shaped case); optional i.i.d. N(0, 1) text tokens prepended
  (CogVideoX-shaped 17.7K case). bf16 workloads are rounded to nearest-even.
  The noise scale 0.1 is the workloads' default; a synthetic stack of layers
  (layer_stack) varies it from layer to layer.

Denoising steps (the warm start of section 3.2.2 relies on tokens moving
little from one step to the next, Fig. 6): step s keeps every field's
amplitude, direction and frequency, advances its phase by s * drift radians,
and draws fresh noise from a sub-stream of its own; text tokens stay fixed.
Step 0 is the plain recipe above.
"""
from __future__ import annotations

import dataclasses
import numpy as np

N_FIELDS = 8
NOISE_STD = 0.1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    D: int
    grid: tuple          # (T, Hg, W) latent grid of video tokens
    text_tokens: int     # i.i.d. N(0,1) tokens prepended to the video tokens
    dtype: str           # "f32" or "bf16"
    q_clusters: int
    k_base: int          # m0: first-stage key cluster count
    k_adaptive: bool     # threshold-adaptive multi-stage key clustering
    iters: int           # Lloyd iterations per k-means call
    init: str            # "kmeanspp" or "sample"
    top_p: float
    noise: str = "normal"        # "normal" | "student_t3" | "student_t" (noise_df degrees of freedom)
    head_scale: bool = False     # per-head U(0.5, 2) scale shared by Q/K/V
    B: int = 1
    noise_std: float = NOISE_STD  # scale of eps (layers of a synthetic stack differ in it)
    noise_df: float = 3.0         # degrees of freedom of the "student_t" noise

    @property
    def N(self) -> int:
        t, h, w = self.grid
        return t * h * w + self.text_tokens

    @property
    def k_max(self) -> int:
        """Nmax: the slot count after three stages of m0, m0, 2 m0."""
        return 4 * self.k_base if self.k_adaptive else self.k_base

    def dense_flops(self) -> float:
        """4 H N^2 D: the flops of dense softmax attention over the same layer."""
        return 4.0 * self.B * self.H * float(self.N) ** 2 * self.D


WORKLOADS = {
    "tiny": Workload("tiny", H=2, D=64, grid=(4, 32, 32), text_tokens=0, dtype="f32",
                     q_clusters=32, k_base=64, k_adaptive=False, iters=5,
                     init="kmeanspp", top_p=0.9),
    "cog17k": Workload("cog17k", H=30, D=64, grid=(13, 30, 45), text_tokens=226,
                       dtype="bf16", q_clusters=256, k_base=256, k_adaptive=True,
                       iters=5, init="sample", top_p=0.9),
    "wan33k": Workload("wan33k", H=12, D=128, grid=(21, 30, 52), text_tokens=0,
                       dtype="bf16", q_clusters=512, k_base=512, k_adaptive=True,
                       iters=5, init="sample", top_p=0.95, head_scale=True),
    "cog76k": Workload("cog76k", H=30, D=64, grid=(21, 45, 80), text_tokens=0,
                       dtype="bf16", q_clusters=1024, k_base=1024, k_adaptive=True,
                       iters=5, init="sample", top_p=0.9),
    "hun119k": Workload("hun119k", H=24, D=128, grid=(33, 45, 80), text_tokens=0,
                        dtype="bf16", q_clusters=2048, k_base=2048, k_adaptive=True,
                        iters=5, init="sample", top_p=0.9, noise="student_t3"),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


def layer_stack(w: Workload, n_layers: int, noise_lo: float = 0.05, noise_hi: float = 0.4,
                df_hi: float = 30.0, df_lo: float = 2.05):
    """A synthetic stack of layers for the per-layer compactness study
    (section 3.2.1, Fig. 4: key distributions differ much between layers):
    layer l has the shape of ``w``, its own fields (input seed l) and Student-t
    noise whose scale grows geometrically from noise_lo to noise_hi while its
    degrees of freedom fall from df_hi to df_lo (2 + geometric in df - 2), so
    later layers are more scattered and heavier-tailed. Returns
    [(workload, seed)] per layer."""
    out = []
    for l in range(n_layers):
        f = l / max(n_layers - 1, 1)
        std = noise_lo * (noise_hi / noise_lo) ** f
        df = 2.0 + (df_hi - 2.0) * ((df_lo - 2.0) / (df_hi - 2.0)) ** f
        out.append((dataclasses.replace(w, noise="student_t", noise_std=float(std), noise_df=float(df)), l))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _tensor_head(rng: np.random.Generator, w: Workload, coords: np.ndarray, step: int = 0,
                 drift: float = 0.0, step_rng: np.random.Generator | None = None) -> np.ndarray:
    """One head of one tensor as float32 [N, D] (before per-head scale / dtype)."""
    T, Hg, W = w.grid
    amp = rng.uniform(0.5, 1.5, size=N_FIELDS)
    dirs = rng.standard_normal((N_FIELDS, w.D))
    kap = rng.uniform(0.0, 2.0, size=(N_FIELDS, 3))
    phi = rng.uniform(0.0, 2.0 * np.pi, size=N_FIELDS) + step * drift
    t, y, x = coords
    phase = 2.0 * np.pi * (np.outer(kap[:, 0], t / T) + np.outer(kap[:, 1], y / Hg)
                           + np.outer(kap[:, 2], x / W)) + phi[:, None]
    field = (np.sin(phase).T @ (amp[:, None] * dirs)).astype(np.float32)   # [Nv, D]
    nv = field.shape[0]
    for g in ((rng,) if step == 0 else (rng, step_rng)):
        # at step > 0 the step-0 draw only advances the base stream (text tokens follow it)
        if w.noise == "student_t3":
            eps = g.standard_t(3, size=(nv, w.D)).astype(np.float32)
        elif w.noise == "student_t":
            eps = g.standard_t(w.noise_df, size=(nv, w.D)).astype(np.float32)
        else:
            eps = g.standard_normal((nv, w.D), dtype=np.float32)
    field += np.float32(w.noise_std) * eps
    if w.text_tokens:
        text = rng.standard_normal((w.text_tokens, w.D), dtype=np.float32)
        field = np.concatenate([text, field], axis=0)
    return field


DRIFT = 0.05   # default phase advance per denoising step, radians


def generate(w: Workload, seed: int = 0, heads=None, step: int = 0, drift: float = DRIFT):
    """Q, K, V for workload ``w`` at denoising step ``step``.

    Returns a dict with ``q``, ``k``, ``v`` of shape [B, H', N, D] where H' is
    ``len(heads)`` (default: all heads). For bf16 workloads the arrays are
    uint16 bfloat16 bit patterns; for f32 workloads they are float32. Each
    (tensor, batch, head) draws from its own PCG64 sub-stream, so a subset of
    heads is bit-identical to the same heads of the full tensor.
    """
    heads = list(range(w.H)) if heads is None else list(heads)
    T, Hg, W = w.grid
    tt, yy, xx = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(W), indexing="ij")
    coords = (tt.ravel().astype(np.float64), yy.ravel().astype(np.float64),
              xx.ravel().astype(np.float64))
    out = {}
    scale_rng = np.random.default_rng([seed, 3])
    head_scales = scale_rng.uniform(0.5, 2.0, size=(w.B, w.H)) if w.head_scale else None
    for ti, name in enumerate(("q", "k", "v")):
        arr = np.empty((w.B, len(heads), w.N, w.D),
                       dtype=np.uint16 if w.dtype == "bf16" else np.float32)
        for b in range(w.B):
            for hi, h in enumerate(heads):
                rng = np.random.default_rng([seed, ti, b, h])
                srng = np.random.default_rng([seed, ti, b, h, step]) if step else None
                x = _tensor_head(rng, w, coords, step, drift, srng)
                if head_scales is not None:
                    x *= np.float32(head_scales[b, h])
                arr[b, hi] = f32_to_bf16_bits(x) if w.dtype == "bf16" else x
        out[name] = arr
    return out


def as_f32(x: np.ndarray) -> np.ndarray:
    """float32 view of a generated tensor (exact for bf16 bit patterns)."""
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float32)
