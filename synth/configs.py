"""Workload table: shapes, dtypes, value recipes and mask parameters.

Every workload is a video latent of ``frames`` frames of ``frame_h x frame_w``
patches flattened frame-major (token t = f * P + h * frame_w + w, P =
frame_h * frame_w), which is the frame-structured sequence the video-diffusion
pages describe (LinVideo page, technical summary section 1: a 10 s video is
more than 50K tokens).  The numeric parameters (window, anchor period, radial
W, cluster counts, density) are the workload definitions this project is
measured on; the pages only describe the shape of each method in prose.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple

MASK_ALL = 0
MASK_WINDOW_ANCHOR = 1
MASK_RADIAL = 2


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    D: int
    frames: int
    frame_h: int
    frame_w: int
    dtype: str                      # "f32" or "bf16": storage and compute-input type
    values: str                     # "iid", "ar1" or "gmm"
    block: int = 128
    # block-mask parameters (None for workloads without a static mask)
    mask_kind: Optional[int] = None
    window: int = 0
    anchor_period: int = 0
    anchor_steps: Tuple[int, ...] = (0,)
    anchor_rows: int = 0
    radial_w: int = 0
    # clustered (SVG-EAR) parameters
    n_q_clusters: int = 0
    n_k_clusters: int = 0
    density_ppm: int = 0
    gmm_sigma: float = 0.3
    kmeans_iters: int = 10
    ar_rho: float = 0.9
    # latent inter-frame pruning (LIPAR): threshold on the mean |difference|
    lipar_tau: float = 0.0
    # which call a workload runs where its values do not say: "causal" or
    # "mixed" (LinVideo blend with weight mix_r on the block-sparse branch) for
    # the linear family, "kmeans" for the token clustering, "bwd" for the
    # block-sparse attention backward
    op: str = ""
    mix_r: float = 0.0
    notes: str = field(default="", compare=False)

    @property
    def P(self) -> int:
        return self.frame_h * self.frame_w

    @property
    def N(self) -> int:
        return self.frames * self.P

    @property
    def nb(self) -> int:
        return -(-self.N // self.block)

    def mask_params(self, step: int = 0) -> dict:
        """Plain dict of mask parameters; each side builds its own descriptor from it."""
        return dict(kind=self.mask_kind, frames=self.frames, frame_tokens=self.P,
                    block=self.block, window=self.window,
                    anchor_period=self.anchor_period, anchor_step=step,
                    anchor_rows=self.anchor_rows, radial_w=self.radial_w)


WORKLOADS = {
    # fp32 correctness case: 4 frames of 8x8, one frame per 64-token block,
    # window |dt| <= 1 plus frame 0 as a row-and-column anchor.
    "tiny_fp32": Workload(
        name="tiny_fp32", seed=0, B=1, H=2, D=64, frames=4, frame_h=8, frame_w=8,
        dtype="f32", values="iid", block=64, mask_kind=MASK_WINDOW_ANCHOR,
        window=1, anchor_period=8, anchor_steps=(0,), anchor_rows=1),
    # LVSA: 21 latent frames of 30x52, key frames within +-3 plus anchor frames
    # every 8th frame whose offset rotates with the denoising step s = 0..3.
    "lvsa_32k": Workload(
        name="lvsa_32k", seed=1, B=1, H=12, D=128, frames=21, frame_h=30, frame_w=52,
        dtype="bf16", values="ar1", block=128, mask_kind=MASK_WINDOW_ANCHOR,
        window=3, anchor_period=8, anchor_steps=(0, 1, 2, 3), anchor_rows=1),
    # The LVSA workload's backward pass (a training step of the attention):
    # same inputs and masks, an N(0,1) output gradient.
    "lvsa_32k_bwd": Workload(
        name="lvsa_32k_bwd", seed=1, B=1, H=12, D=128, frames=21, frame_h=30, frame_w=52,
        dtype="bf16", values="ar1", block=128, mask_kind=MASK_WINDOW_ANCHOR,
        window=3, anchor_period=8, anchor_steps=(0, 1, 2, 3), anchor_rows=1, op="bwd"),
    # Radial: 126 latent frames (6x horizon), spatial band W / 2^floor(log2|dt|).
    "radial_196k": Workload(
        name="radial_196k", seed=2, B=1, H=12, D=128, frames=126, frame_h=30, frame_w=52,
        dtype="bf16", values="ar1", block=128, mask_kind=MASK_RADIAL, radial_w=1560),
    # SVG-EAR: Gaussian-mixture Q/K, tokens ordered by k-means cluster, 15% density.
    "svg_ear_32k": Workload(
        name="svg_ear_32k", seed=3, B=1, H=12, D=128, frames=21, frame_h=30, frame_w=52,
        dtype="bf16", values="gmm", n_q_clusters=100, n_k_clusters=500,
        density_ppm=150000),
    # Token clustering in front of SVG-EAR: the same inputs as svg_ear_32k in
    # token order, k-means of queries (100 clusters) and keys (500), 10 steps
    # each from the generating centres, then the rows into cluster order.
    "kmeans_32k": Workload(
        name="kmeans_32k", seed=3, B=1, H=12, D=128, frames=21, frame_h=30, frame_w=52,
        dtype="bf16", values="gmm", n_q_clusters=100, n_k_clusters=500,
        density_ppm=150000, op="kmeans"),
    # LinVideo-style elu+1 linear attention at two lengths.
    "linear_32k": Workload(
        name="linear_32k", seed=4, B=1, H=12, D=128, frames=21, frame_h=30, frame_w=52,
        dtype="bf16", values="iid"),
    # Causal (chunked) elu+1 linear attention, the 32,760-token latent.
    "causal_linear_32k": Workload(
        name="causal_linear_32k", seed=7, B=1, H=12, D=128, frames=21, frame_h=30, frame_w=52,
        dtype="bf16", values="iid", op="causal"),
    # LinVideo mixed attention: r = 0.5 of the LVSA block-sparse branch (mask as
    # lvsa_32k) plus 0.5 of elu+1 linear attention.
    "mixed_32k": Workload(
        name="mixed_32k", seed=8, B=1, H=12, D=128, frames=21, frame_h=30, frame_w=52,
        dtype="bf16", values="ar1", block=128, mask_kind=MASK_WINDOW_ANCHOR,
        window=3, anchor_period=8, anchor_steps=(0, 1, 2, 3), anchor_rows=1, op="mixed", mix_r=0.5),
    "linear_196k": Workload(
        name="linear_196k", seed=5, B=1, H=12, D=128, frames=126, frame_h=30, frame_w=52,
        dtype="bf16", values="iid"),
    # LIPAR: one latent token sequence of 21 frames x 30x52 patches, 1536 values
    # per token (a DiT hidden width); a static scene with per-frame jitter, a
    # moving object and a region that changes every frame (the "video" recipe).
    "lipar_32k": Workload(
        name="lipar_32k", seed=6, B=1, H=1, D=1536, frames=21, frame_h=30, frame_w=52,
        dtype="bf16", values="video", lipar_tau=0.05),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
