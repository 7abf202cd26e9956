"""Workload shapes for the FLUX.3 Image Klein parallel DiT block.

Shapes follow "Welcome FLUX.3 Image Klein in Diffusers", section "How it works":
a 1024x1024 image is 4,096 latent tokens (one token per 16x16 pixels), prompts
are padded to a multiple of 80 tokens, the width is 3072 with 24 heads of 128,
stage 1 has 5 blocks per stream and stage 2 has 28 shared joint blocks.  The
SwiGLU hidden size (9216 = 3 x width) is not printed on the pages; it is the
reading adopted here (it makes the transformer about 5.3B parameters, close to
the 5.6B the NeMo AutoModel page lists under "Model Architecture").

Token order inside one sequence is always [image | reference | text].
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

WIDTH = 3072
N_HEADS = 24
HEAD_DIM = 128
MLP_HIDDEN = 9216
ROPE_THETA = 10000.0
LN_EPS = 1e-6
QK_EPS = 1e-6

STREAM_IMAGE = "image"
STREAM_REF = "reference"
STREAM_TEXT = "text"


@dataclass(frozen=True)
class Stream:
    """One segment of the joint sequence.

    kind: image / reference / text.
    n: token count.
    grid: (rows, cols) of the latent grid for image and reference streams.
    t: the timestep label of this stream's modulation (image tokens carry the
       current t, text and reference tokens always t=0); it only keys the
       seeded draw of the modulation vectors.
    """

    kind: str
    n: int
    grid: Tuple[int, int] = (0, 0)
    t: float = 0.0


@dataclass(frozen=True)
class BlockConfig:
    name: str
    config_id: int
    streams: Tuple[Stream, ...]
    width: int = WIDTH
    n_heads: int = N_HEADS
    head_dim: int = HEAD_DIM
    mlp_hidden: int = MLP_HIDDEN
    description: str = ""

    @property
    def n_tokens(self) -> Tuple[int, ...]:
        return tuple(s.n for s in self.streams)

    @property
    def N(self) -> int:
        return sum(s.n for s in self.streams)

    @property
    def n_streams(self) -> int:
        return len(self.streams)

    def gemm_flop(self) -> float:
        D, F = self.width, self.mlp_hidden
        # input projection [N,D] x [D, 3D+2F] and output projection [N, D+F] x [D+F, D]
        return 2.0 * self.N * D * (3 * D + 2 * F) + 2.0 * self.N * (D + F) * D

    def attn_flop(self) -> float:
        # QK^T and PV, each 2*N*N*d per head
        return 4.0 * self.N * self.N * self.head_dim * self.n_heads

    def flop(self) -> float:
        return self.gemm_flop() + self.attn_flop()


def _img(n_side: int, t: float) -> Stream:
    return Stream(STREAM_IMAGE, n_side * n_side, (n_side, n_side), t)


def _ref(n_side: int) -> Stream:
    return Stream(STREAM_REF, n_side * n_side, (n_side, n_side), 0.0)


def _txt(n: int) -> Stream:
    return Stream(STREAM_TEXT, n, (0, 0), 0.0)


C1 = BlockConfig(
    "c1", 1, (_img(16, 0.7), _txt(80)),
    description="tiny joint block: 16x16 image (256 tokens, t=0.7) + 80 text tokens, N=336")
C2 = BlockConfig(
    "c2", 2, (_img(64, 0.7), _txt(160)),
    description="1024^2 joint block: 64x64 image (4096 tokens) + 160 text tokens, N=4256")
C3_IMG = BlockConfig(
    "c3_img", 3, (_img(64, 0.9),),
    description="stage-1 image-only block: 4096 tokens at t=0.9")
C3_TXT = BlockConfig(
    "c3_txt", 4, (_txt(80),),
    description="stage-1 text-only block: 80 tokens at t=0")
C4 = BlockConfig(
    "c4", 5, (_img(64, 0.5), _ref(64), _txt(160)),
    description="1024^2 with one 1024^2 reference: 4096 + 4096 (l=1) + 160 text, N=8352")

# Long editing sequence: a 2048^2 image (a 128 x 128 latent grid) with one
# 2048^2 reference and 160 text tokens, N = 32,928; attention is about 60% of
# its FLOPs.
EDIT_2048 = BlockConfig(
    "edit2048", 6, (_img(128, 0.5), _ref(128), _txt(160)),
    description="2048^2 edit: 16384 image + 16384 reference (l=1) + 160 text, N=32928")

CONFIGS = {c.name: c for c in (C1, C2, C3_IMG, C3_TXT, C4, EDIT_2048)}


@dataclass(frozen=True)
class StackConfig:
    """Two-stage DiT stack for one denoise step (stage 1 per stream, stage 2 joint)."""

    name: str = "c5"
    n_stage1: int = 5
    n_joint: int = 28
    image_side: int = 64
    n_text: int = 160
    cfg_scale: float = 4.0
    t: float = 0.7
    stage1_blocks: Tuple[str, ...] = field(default=("image", "text"))


C5 = StackConfig()
