"""Workload shapes for the DFlash KV-injection block drafter.

Each entry fixes the drafter geometry, the borrowed target's hidden size and
vocabulary, the draft length gamma, the context length and the weight format.

Geometry sources (pages named by title and section):
  * "Faithful DFlash drafter" (mlx-bun inference diff, dflash.ts):
    DEFAULT_DFLASH_CONFIG gives gamma 5, draft width 1024, 5 layers, 8 heads,
    FFN multiplier 2 and four taps; the FFN there is gated GELU.
  * "Inco Hacks Native: DFlash 2 Speculation", section 1 (Architectural
    Geometry): block 8 = 1 verify + 7 proposals, 5 taps, hidden 5120,
    intermediate 17408, head dim 128, a 4-bit quantised drafter.
  * The 40 query / 8 key-value head split, SwiGLU for the wide drafter, the
    context lengths, the vocabularies and the 4-bit group layout are workload
    choices of this library (the pages do not print them).

gamma is the number of block query rows and of drafted tokens; the verify
width is gamma + 1 (anchor row plus gamma drafts).
"""

from dataclasses import dataclass, replace
from typing import Optional, Tuple

WDTYPE_F32 = "f32"
WDTYPE_BF16 = "bf16"
WDTYPE_INT4G64 = "int4g64"

ACT_GELU_TANH = "gelu_tanh"
ACT_SILU = "silu"

GROUP = 64  # int4 quantisation group along the reduction axis


@dataclass(frozen=True)
class Dims:
    name: str
    H: int          # target hidden size (tap width, LM-head width)
    m: int          # number of tapped target layers
    d: int          # drafter width
    nl: int         # drafter layers
    hq: int         # query heads
    hkv: int        # key/value heads
    hd: int         # head dim
    F: int          # FFN inner width
    act: str        # FFN activation on the gate branch
    gamma: int      # block query rows = drafted tokens
    L: int          # context rows (per sequence; the minimum for ragged batches)
    V: int          # vocabulary
    B: int          # sequences
    wdtype: str     # weight format
    eps: float = 1e-6
    L_max: Optional[int] = None   # ragged batches: lengths drawn from [L, L_max]
    r: int = 0                    # rank of the DSpark sequential (Markov) head; 0 = no head
    window: int = 0               # DFlash2: context keys attended, from the end; 0 = all
    rope_theta: float = 0.0       # DFlash2: rotary base; 0 = no rotary positions
    verify: str = "logits"        # what the target hands the verify: "logits" or "hidden" states

    @property
    def qkv_rows(self) -> int:
        return (self.hq + 2 * self.hkv) * self.hd

    @property
    def kv_width(self) -> int:
        return self.hkv * self.hd

    @property
    def fp32(self) -> bool:
        return self.wdtype == WDTYPE_F32


TINY = Dims("tiny", H=256, m=2, d=128, nl=2, hq=2, hkv=2, hd=64, F=256,
            act=ACT_GELU_TANH, gamma=4, L=32, V=512, B=1, wdtype=WDTYPE_F32)

DEFAULT = Dims("default", H=2560, m=4, d=1024, nl=5, hq=8, hkv=8, hd=128, F=2048,
               act=ACT_GELU_TANH, gamma=5, L=2048, V=32768, B=1, wdtype=WDTYPE_BF16)

WIDE = Dims("wide", H=5120, m=5, d=5120, nl=5, hq=40, hkv=8, hd=128, F=17408,
            act=ACT_SILU, gamma=7, L=4096, V=151936, B=1, wdtype=WDTYPE_BF16)

WIDE4 = Dims("wide4", H=5120, m=5, d=5120, nl=5, hq=40, hkv=8, hd=128, F=17408,
             act=ACT_SILU, gamma=4, L=8192, V=151936, B=1, wdtype=WDTYPE_INT4G64)

BATCHED = Dims("batched", H=5120, m=5, d=5120, nl=5, hq=40, hkv=8, hd=128, F=17408,
               act=ACT_SILU, gamma=7, L=8192, V=151936, B=16, wdtype=WDTYPE_BF16,
               L_max=16384)

# The DFlash2 drafter (page "Inco Hacks Native: DFlash 2 Speculation", section 1): the wide
# geometry in 4-bit weights, block 8 (gamma 7), a sliding window over the context, rotary
# positions, and a verify that scores the target's hidden states with the borrowed head. The
# page gives neither the window nor the rotary base: 2048 keys and base 1e6 (the Qwen3
# family's) are this library's choices.
DFLASH2 = Dims("dflash2", H=5120, m=5, d=5120, nl=5, hq=40, hkv=8, hd=128, F=17408,
               act=ACT_SILU, gamma=7, L=8192, V=151936, B=1, wdtype=WDTYPE_INT4G64,
               window=2048, rope_theta=1e6, verify="hidden")

CONFIGS = {c.name: c for c in (TINY, DEFAULT, WIDE, WIDE4, BATCHED, DFLASH2)}


def scaled(base: Dims, **kw) -> Dims:
    """A copy of a config with some fields replaced (small parity shapes)."""
    return replace(base, **kw)
