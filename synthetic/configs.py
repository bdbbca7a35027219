"""The five workload configurations (shapes, tiling, routing, dtypes).

Model shapes stand in for the models the pages evaluate on (their weights and
datasets are not available): Qwen3-8B attention = 32 query / 8 KV heads with
head dim 128; Gemma-3-12B = 16 / 8 heads with head dim 256; the 32k sequence
stands in for long-context evaluation.
"""
from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    causal: bool
    dtype: str                    # "f16" | "bf16"
    tile_m: int
    tile_n: int
    tiles_per_bit: int
    frac_16bit: float             # fraction of groups on the 16-bit path
    code: str                     # "i8" | "e4m3"
    exp8: bool
    adaptive: bool = False
    tau: float = 4.0
    sub_rows: int = 32
    outliers: bool = False        # 4 x20 outlier channels + sink key 0
    input_seed: int = 0
    mask_seed: int = 0
    mask_all_ones: bool = False   # adaptive config routes every tile 8-bit first
    sm_scale: float = 0.0         # <= 0 -> 1/sqrt(D)
    input_scale: float = 1.0      # Q and K multiplied by this (fp32, before the cast)

    @property
    def n_qt(self):
        return -(-self.S // self.tile_m)

    @property
    def n_kt(self):
        return -(-self.S // self.tile_n)

    @property
    def n_g(self):
        return -(-self.n_kt // self.tiles_per_bit)

    @property
    def words_per_row(self):
        return -(-self.n_g // 64)

    def with_(self, **kw):
        return replace(self, **kw)

    def fa_flops(self):
        """FlashAttention-convention flops: 4 B Hq S^2 D (halved if causal)."""
        f = 4.0 * self.B * self.Hq * self.S * self.S * self.D
        return f / 2 if self.causal else f


C1 = Config("tiny_exact_256", B=1, Hq=1, Hkv=1, S=256, D=64, causal=False, dtype="f16",
            tile_m=64, tile_n=64, tiles_per_bit=1, frac_16bit=0.5, code="i8", exp8=False,
            input_seed=1001, mask_seed=2001)
C2 = Config("qwen3_8b_4k", B=1, Hq=32, Hkv=8, S=4096, D=128, causal=True, dtype="bf16",
            tile_m=128, tile_n=64, tiles_per_bit=4, frac_16bit=0.25, code="i8", exp8=False,
            input_seed=1002, mask_seed=2002)
C3 = Config("gemma3_12b_8k_adaptive", B=1, Hq=16, Hkv=8, S=8192, D=256, causal=True,
            dtype="bf16", tile_m=128, tile_n=64, tiles_per_bit=1, frac_16bit=0.0,
            code="e4m3", exp8=True, adaptive=True, tau=4.0, sub_rows=32, outliers=True,
            input_seed=1003, mask_seed=2003, mask_all_ones=True)
C4 = Config("long_32k_int8", B=1, Hq=32, Hkv=8, S=32768, D=128, causal=True, dtype="bf16",
            tile_m=128, tile_n=64, tiles_per_bit=8, frac_16bit=0.10, code="i8", exp8=False,
            input_seed=1004, mask_seed=2004)
C5 = Config("qwen3_8b_16k_mix", B=2, Hq=32, Hkv=8, S=16384, D=128, causal=True, dtype="bf16",
            tile_m=128, tile_n=64, tiles_per_bit=4, frac_16bit=0.25, code="i8", exp8=False,
            input_seed=1005, mask_seed=2005)

C5_FRACS = (0.0, 0.10, 0.25, 0.50, 1.0)

CONFIGS = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}


def c5_variant(frac_16bit, code="i8"):
    """One point of the precision-mix sweep: int8 (TileMix, exp8 off) or
    e4m3 (8-bit exp on) at a given 16-bit fraction, same inputs."""
    return C5.with_(frac_16bit=frac_16bit, code=code, exp8=(code == "e4m3"),
                    mask_seed=2005 + int(100 * frac_16bit + 1e-9),
                    name=f"qwen3_8b_16k_mix_f{int(round(100 * frac_16bit)):02d}_{code}")


def get_config(name: str, frac_16bit: Optional[float] = None, code: Optional[str] = None):
    if name == "C5" and (frac_16bit is not None or code is not None):
        return c5_variant(0.25 if frac_16bit is None else frac_16bit, code or "i8")
    return CONFIGS[name]
