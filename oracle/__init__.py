"""Oracle: plain, slow, float64 CPU reference for exact tiled attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The product path (``exact_tiled_attention_31_amd``) never imports it, and the
oracle imports nothing from the product path: the two share no code.  The
only module both sides use is ``workloads`` (seeded input generation, which
holds none of the method's arithmetic).

Pages cited (each by title and section):
  * "How FlashAttention Uses Tiling" (mbrenndoerfer.com) -- softmax, the
    running statistics and their update equations, the two-block intuition.
  * "FlashAttention" (attention-lab explainer, divagr.pages.dev) -- tiled
    computation with running max/sum/output; the cost assumptions.
  * "LLM Architecture Refresh [3]: Flash Attention Is Exact, and Here's the
    Proof" -- sections 1-8 (standard attention, online softmax, the tiled
    loop, causal skipping, the flop/byte counters).

Contents:
  attention      -- the definition softmax(scale*Q K^T + mask) V, its
                    log-sum-exp, and its gradient (float64, numpy).
  online_softmax -- the streaming normaliser with its per-block trace.
  tiled          -- the tiled loop (float64) with the pages' counters, the
                    closed-form tile counts, and the sliding-window
                    negative control.

Every function here is pinned by ``tests/test_oracle_*.py`` against values
the pages print, closed forms, invariants or brute force.  No function is
"parity unpinned".
"""
from .attention import (attention_fwd, attention_rows, attention_bwd,
                        attention_probs, kv_head_of)
from .online_softmax import online_normaliser, online_softmax, softmax_direct
from .tiled import (tiled_attention, causal_tile_counts, tile_counts, naive_counts,
                    sliding_window_attention)

__all__ = [
    "attention_fwd", "attention_rows", "attention_bwd", "attention_probs",
    "kv_head_of", "online_normaliser", "online_softmax", "softmax_direct",
    "tiled_attention", "causal_tile_counts", "tile_counts", "naive_counts",
    "sliding_window_attention",
]
