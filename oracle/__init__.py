"""CPU oracle of the DeepSeek sparse-attention (DSA) decode path.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import, call or run anything in this package; the HIP path
(sparse_attention_14_amd/) never does, and this package imports nothing from it.
The two share no code: inputs come from the seeded generator in workloads.py.

Plain, slow, obviously-correct numpy.  Floating point is float64 throughout, except
the activation quantizer, whose precision the pages fix at fp32 (the quant operator
converts its input to fp32 before taking the row max and dividing by the scale).

Sources (cited by page title and section; no line numbers):
  [SFA]   "NPU DeepSeek-V4 TileLang算子开发实践" (mooersco.com/news/996258),
          section 1 "Sparse Flash Attention", algorithm steps 1-8.
  [AQ]    same page, section 4 "Activation Quantization", steps 1-4.
  [PRO]   "NPU DeepSeek-V3.2-Exp PyPTO 融合算子开发优化实践" (jsqmd.com/news/787325),
          "Indexer Prolog", formulas and quant strategy.
  [LI]    same page, "Lightning Indexer" (scores -> TopK).
  [DIA]   same page, "Deepseek Indexer Attention" (the four-part decode layer); the Page
          Attention cache blocks of the Lightning Indexer analysis (paged.py).

Parity status of each function is stated in its docstring; every function here is
pinned by CPU tests in tests/test_oracle_*.py except where it says "parity unpinned".
"""
from .formats import (bf16_encode, bf16_decode, e4m3_encode, e4m3_decode, fp16_round)
from .prolog import hadamard, apply_rope, quantize_rows, prolog_rows, indexer_prolog
from .indexer import indexer_dots, indexer_scores
from .topk import topk_select
from .sfa import sparse_attention
from .step import decode_step
from .paged import paged_rows, flatten_paged
from .projections import w8a8_dequant, linear, layer_norm, indexer_projections

__all__ = ["bf16_encode", "bf16_decode", "e4m3_encode", "e4m3_decode", "fp16_round",
           "hadamard", "apply_rope", "quantize_rows", "prolog_rows", "indexer_prolog",
           "indexer_dots", "indexer_scores", "topk_select", "sparse_attention", "decode_step",
           "w8a8_dequant", "linear", "layer_norm", "indexer_projections"]
