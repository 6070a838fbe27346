"""CPU oracle of the batch-1 MLA + MoE decode step (float64, numpy).

TEST INFRASTRUCTURE ONLY. This package is the independent reference that the
HIP engine is checked against. Only the tests, the smoke check of the package
entry point and the benchmark's CPU-baseline leg may import or run it; the
engine's own code path never does, and the oracle shares no code with the
engine (the seeded input generators under `synth` are the only common part).

Every function states the passage of the TileRT pages it follows, or the
reading chosen where the pages are silent. Parity pins (tests under tests/
marked "not gpu") tie each function to closed forms, library routines,
brute force or invariants. No function here is "parity unpinned".
"""
from . import numerics, model, batch  # noqa: F401
from .numerics import (E2M1, E4M3, bf16_round, bf16_bits_to_f64, dequant_fp8, dequant_mxfp4,  # noqa: F401
                       e2m1_decode, e4m3_decode, e8m0_decode)
from .model import (OracleWeights, DecodeState, decode_step, forward_full, prefill,  # noqa: F401
                    rmsnorm, rope, softmax, route, topk_indices, mla_absorbed, mla_naive,
                    split_wkv_b, attention_decode, ffn_decode, lm_logits)
from .batch import batch_gemm, batch_ffn  # noqa: F401
from . import dsa  # noqa: F401
