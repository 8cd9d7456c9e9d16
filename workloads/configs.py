"""The five synthetic decode-step workloads (shapes, sizes, value distributions).

Plain data, no arithmetic of the method.  The shapes follow the "Optimized
Parler TTS" page: a 24-layer MusicGen-style decoder with d_model 1024 and 16
heads of 64 ("A rough architecture of Parler TTS"), 9 DAC codebooks emitted per
step under a delay pattern (same section), a 1089-entry codebook vocabulary
padded to a multiple of 8 ("Analysis and improvements", item 4), and the two
end-to-end regimes the page measures (1024 description tokens with 1024 output
tokens; 64 description tokens with 2048 output tokens; "Analysis and
improvements", the batch-size-1 results).
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

N_CODEBOOKS = 9          # DAC codebooks decoded in parallel per step
VOCAB_VALID = 1089       # codebook vocabulary before padding
VOCAB_PADDED = 1096      # next multiple of 8
SEED_ROOT = 20261202     # root of every SeedSequence used by the generators


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    n_layers: int
    batch: int
    heads: int
    head_dim: int
    dtype: str                      # "bf16" or "f32": element type of q, K, V
    self_cap: int                   # static self-attention cache capacity (slots)
    cross_cap: int                  # static cross-attention (description) capacity
    self_len: Optional[int]         # fixed valid self length (None: drawn per sequence)
    cross_len: Optional[int]        # fixed valid cross length (None: drawn per sequence)
    self_len_range: Optional[Tuple[int, int]] = None   # inclusive range when drawn
    cross_len_range: Optional[Tuple[int, int]] = None
    qkv_std: float = 0.125          # N(0,1)/sqrt(64)
    cross_kv_std: float = 0.125
    logit_std: float = 3.0
    vocab_valid: int = VOCAB_VALID
    vocab_stride: int = VOCAB_PADDED
    n_codebooks: int = N_CODEBOOKS
    top_k: int = 50
    temperature: Optional[float] = 1.0                  # fixed T, or None: drawn per sequence
    temperature_range: Optional[Tuple[float, float]] = None
    n_steps: int = 1                # successive decode steps (long-output workload)
    delay: bool = False             # apply the codebook delay mask in the step
    fill_token: int = VOCAB_VALID   # token emitted by a codebook that has not started yet
    scale: float = 0.125            # attention scale 1/sqrt(head_dim)


TINY = Workload(
    cfg_id=1, name="tiny", n_layers=1, batch=1, heads=4, head_dim=64, dtype="f32",
    self_cap=256, cross_cap=16, self_len=37, cross_len=16,
    vocab_valid=VOCAB_VALID, vocab_stride=VOCAB_VALID)

MINI_V1 = Workload(
    cfg_id=2, name="mini_v1", n_layers=24, batch=1, heads=16, head_dim=64, dtype="bf16",
    self_cap=4096, cross_cap=64, self_len=1024, cross_len=64)

LONG_DESCRIPTION = Workload(
    cfg_id=3, name="long_description", n_layers=24, batch=1, heads=16, head_dim=64,
    dtype="bf16", self_cap=4096, cross_cap=1024, self_len=64, cross_len=1024,
    cross_kv_std=1.0)

LONG_OUTPUT = Workload(
    cfg_id=4, name="long_output", n_layers=24, batch=1, heads=16, head_dim=64, dtype="bf16",
    self_cap=4096, cross_cap=64, self_len=2048, cross_len=64, n_steps=2048, delay=True)

BATCHED = Workload(
    cfg_id=5, name="batched_mixed", n_layers=24, batch=32, heads=16, head_dim=64,
    dtype="bf16", self_cap=4096, cross_cap=512, self_len=None, cross_len=None,
    self_len_range=(64, 2048), cross_len_range=(16, 512),
    temperature=None, temperature_range=(0.7, 1.3))

ALL = (TINY, MINI_V1, LONG_DESCRIPTION, LONG_OUTPUT, BATCHED)
BY_ID = {w.cfg_id: w for w in ALL}
BY_NAME = {w.name: w for w in ALL}

# Stream ids inside the seed tuple (SEED_ROOT, cfg_id, stream, layer, index, step).
STREAM_Q_SELF, STREAM_K_SELF, STREAM_V_SELF = 0, 1, 2
STREAM_Q_CROSS, STREAM_K_CROSS, STREAM_V_CROSS = 3, 4, 5
STREAM_LENGTHS, STREAM_LOGITS, STREAM_UNIFORMS, STREAM_TEMPERATURE = 6, 7, 8, 9
STREAM_K_NEW, STREAM_V_NEW = 10, 11           # the current token's key/value rows per step
STREAM_HIDDEN, STREAM_LM_W, STREAM_EMBED = 12, 13, 14   # LM head input / weights, embeddings
D_MODEL = 1024                 # decoder width (24 layers x 16 heads x 64)


def valid_kv_bytes(w: Workload, self_lens, cross_lens) -> int:
    """Bytes of K and V inside the valid prefixes (the only cache bytes a step must read)."""
    elem = 2 if w.dtype == "bf16" else 4
    per_row = 2 * w.heads * w.head_dim * elem * w.n_layers     # K + V, all layers and heads
    s = sum(min(max(int(n), 0), w.self_cap) for n in self_lens)
    c = sum(min(max(int(n), 0), w.cross_cap) for n in cross_lens)
    return per_row * (s + c)
