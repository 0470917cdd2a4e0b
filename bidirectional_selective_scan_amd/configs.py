"""The five seeded synthetic workloads of the bidirectional selective scan.

Shapes follow the vision-Mamba settings the source pages discuss:
- "tiny": 8x8 patches plus a middle class token (L=65), a toy channel count;
- "vim_ti": 14x14 patches plus the class token (L=197), Vim-Ti's inner width 384;
- "vim_s": the same token count at Vim-S's inner width 768 (the headline shape);
- "highres": a 512x512 image at patch 16 (32x32 patches plus class token, L=1025);
- "folded": 256 sequences of 7x7 patches plus two auxiliary head/tail tokens (L=51) folded into
  one stream of 13056 tokens with a state reset every 51 tokens (SF-Mamba, "Batch folding and
  periodic state reset").

The class token and the auxiliary tokens are ordinary tokens to the scan (Vim page, section 2.3;
SF-Mamba page, "Auxiliary patch swap"), so only the token count L enters here.
"""
from __future__ import annotations

from dataclasses import dataclass

D_STATE = 16


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    d_inner: int
    seg_len: int  # 0: no internal reset; else a reset every seg_len tokens
    io_dtype: str  # "f32" or "bf16": dtype of x, dt, z, B_*, C_* and y
    seed: int = 0
    d_state: int = D_STATE

    @property
    def tokens_channels(self) -> int:
        return self.batch * self.seqlen * self.d_inner

    @property
    def io_bytes(self) -> int:
        return 4 if self.io_dtype == "f32" else 2

    def algorithmic_bytes(self) -> int:
        """Bytes the scan must move: read x, dt, z, B_f, C_f, B_b, C_b once, the fp32
        parameters A_f, A_b, D_f, D_b, dt_bias_f, dt_bias_b once, and write y once."""
        e = self.io_bytes
        s = self.tokens_channels
        bc = 4 * self.batch * self.seqlen * self.d_state * e
        params = (2 * self.d_inner * self.d_state + 4 * self.d_inner) * 4
        return s * (3 * e + e) + bc + params

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "batch": self.batch,
            "seqlen": self.seqlen,
            "d_inner": self.d_inner,
            "d_state": self.d_state,
            "seg_len": self.seg_len,
            "io_dtype": self.io_dtype,
        }


WORKLOADS = [
    Workload("tiny_b2_l65_d32_f32", 2, 65, 32, 0, "f32"),
    Workload("vim_ti_b64_l197_d384_f32", 64, 197, 384, 0, "f32"),
    Workload("vim_s_b128_l197_d768_bf16", 128, 197, 768, 0, "bf16"),
    Workload("highres_b8_l1025_d768_bf16", 8, 1025, 768, 0, "bf16"),
    Workload("folded_256x51_d1536_bf16", 1, 13056, 1536, 51, "bf16"),
]

# The workload the throughput metric is quoted on: Vim-S (batch 128, L=197, d_inner 768).
HEADLINE = 2
