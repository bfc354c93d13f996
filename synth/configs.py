"""Workload shapes for the FLUX.3 Image Klein transformer block.

Shapes follow the release pages: width 3072 with 24 heads of 128 ("Inside the
transformer", rohitghumare.com guide); one token per 16x16 pixel patch, so a
1024x1024 image is a 64x64 grid of 4096 tokens and a 4096x4096 image is 65536
tokens ("The latent space and the VAE", same guide); prompts padded to a
multiple of 80 tokens ("Speed, architecture, and how the tokens move",
15jq.com post); a 1024x1024 reference adds 4096 tokens to every call (same
section).  The SwiGLU hidden width 9216 is the ratio-3 reading that makes the
published parameter count 5,538,458,368 come out exactly ("What step
distillation removed", rohitghumare.com guide).

Only sizes and segment bookkeeping live here: position ids and every other
piece of the block's arithmetic are computed separately by the oracle and by
the HIP kernels.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

MODE_TEXT, MODE_IMAGE, MODE_REF = 0, 1, 2


@dataclass(frozen=True)
class Dims:
    width: int = 3072
    heads: int = 24
    head_dim: int = 128
    mlp_hidden: int = 9216


DIMS = Dims()


@dataclass(frozen=True)
class Segment:
    start: int
    count: int
    mode: int


@dataclass(frozen=True)
class RopeLayout:
    """Token layout of one call: text, then the noisy-image grid, then refs.

    ``refs`` lists each reference's token grid as (rows, cols).  ``hw_scale``
    is the factor applied to a grid row/col to get its h/w position (0.5 is
    the row/2, col/2 reading of the position table); ``theta`` is the RoPE
    base.
    """
    n_text: int
    grid_h: int
    grid_w: int
    refs: Tuple[Tuple[int, int], ...] = ()
    theta: float = 10000.0
    hw_scale: float = 0.5

    @property
    def n_image(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def n_tokens(self) -> int:
        return self.n_text + self.n_image + sum(h * w for h, w in self.refs)

    def segments(self) -> List[Segment]:
        segs, start = [], 0
        if self.n_text:
            segs.append(Segment(start, self.n_text, MODE_TEXT))
            start += self.n_text
        if self.n_image:
            segs.append(Segment(start, self.n_image, MODE_IMAGE))
            start += self.n_image
        for h, w in self.refs:
            segs.append(Segment(start, h * w, MODE_REF))
            start += h * w
        return segs


@dataclass(frozen=True)
class Workload:
    name: str
    layout: RopeLayout
    description: str
    t_image: float = 0.5
    stack: bool = True
    tags: Tuple[str, ...] = field(default_factory=tuple)

    @property
    def n_tokens(self) -> int:
        return self.layout.n_tokens


WORKLOADS = {
    # 80 text + 16x16 grid (256x256 px): one joint block, the small case.
    "block336": Workload("block336", RopeLayout(80, 16, 16),
                         "80 text + 16x16 image tokens (256x256 px)", t_image=0.5),
    # 1024x1024 text-to-image: 240 padded text tokens + 64x64 image grid.
    "t2i4336": Workload("t2i4336", RopeLayout(240, 64, 64),
                        "240 text + 64x64 image tokens (1024x1024 px)"),
    # Per-mode stage alone: a 240-token text stream and a 4096-token image stream.
    "permode_text240": Workload("permode_text240", RopeLayout(240, 0, 0),
                                "240-token text stream, per-mode blocks only"),
    "permode_image4096": Workload("permode_image4096", RopeLayout(0, 64, 64),
                                  "64x64 image stream, per-mode blocks only"),
    # Single-reference edit: [240 text | 4096 image | 4096 reference].
    "edit8432": Workload("edit8432", RopeLayout(240, 64, 64, ((64, 64),)),
                         "240 text + 64x64 image + 64x64 reference tokens"),
    # 4K text-to-image: 240 text + 256x256 image grid (4096x4096 px).
    "t2i4k65776": Workload("t2i4k65776", RopeLayout(240, 256, 256),
                           "240 text + 256x256 image tokens (4096x4096 px)"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]
