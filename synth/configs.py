"""The five synthetic workloads, as plain data.

Shapes follow the pages' workloads:
  * "tiny"  - a CPU-checkable fp32 layer (2 reused segments + a short suffix).
  * "32k"   - six reused 5000-token segments and a 64-token question, the shape
              of the HotpotQA-distractor RAG demo (RedKnot tutorial page,
              "step 2: run the demo": 6 segments x 5000 tokens, ~15 % global
              heads, the rest local with window 256 when no head config is given).
  * "16k"   - 4 x 4096-token segments, the 16K "4x4K" Qwen3-32B comparison
              (same tutorial, "advanced usage" table).
  * "128k"  - the 128K point of the SegPagedAttention microbenchmark (same table).
  * "batch" - a 32-sequence serving mix (product page, section 6: concurrency).

Nothing here computes anything of the method: these are the knobs the
generator in ``synth.generate`` turns into concrete inputs.
"""

# Class codes shared with the C header (SP_GLOBAL, SP_LOCAL, SP_RETRIEVAL, SP_DENSE).
GLOBAL, LOCAL, RETRIEVAL, DENSE = 0, 1, 2, 3
CLASS_NAMES = {GLOBAL: "global", LOCAL: "local", RETRIEVAL: "retrieval", DENSE: "dense"}

CONFIGS = {
    "tiny": dict(
        idx=0, n_layers=1, n_kv=4, group=1, head_dim=64, dtype="f32", page_size=16,
        theta=10000.0, k_scale=1.0,
        # explicit per-slot classes: head 0 global, heads 1-3 local (window 64)
        slot_classes=[(GLOBAL, 0), (LOCAL, 64), (LOCAL, 64), (LOCAL, 64)],
        seqs=dict(kind="fixed", seg_lens=[256, 256], offline=[0, 0]),
        n_prefill=32, n_decode=1,
    ),
    "32k": dict(
        idx=1, n_layers=8, n_kv=8, group=4, head_dim=128, dtype="bf16", page_size=16,
        theta=10000.0, k_scale=0.5,
        # (class, percent, window, retrieval pages) in the order the mix is stated
        mix=[(GLOBAL, 15, 0, 0), (LOCAL, 85, 256, 0)],
        seqs=dict(kind="fixed", seg_lens=[5000] * 6, offline=[0] * 6),
        n_prefill=64, n_decode=1,
    ),
    "16k": dict(
        idx=2, n_layers=8, n_kv=8, group=8, head_dim=128, dtype="bf16", page_size=16,
        theta=10000.0, k_scale=1.0,
        mix=[(LOCAL, 90, 512, 0), (GLOBAL, 5, 0, 0), (RETRIEVAL, 3, 0, 64), (DENSE, 2, 0, 0)],
        seqs=dict(kind="fixed", seg_lens=[4096] * 4, offline=[0] * 4),
        n_prefill=128, n_decode=1,
    ),
    "128k": dict(
        idx=3, n_layers=8, n_kv=8, group=4, head_dim=128, dtype="bf16", page_size=32,
        theta=10000.0, k_scale=1.0,
        mix=[(LOCAL, 90, 1024, 0), (GLOBAL, 10, 0, 0)],
        # one reused 129024-token segment whose keys were cached 4096 positions
        # earlier than where they are reused (offline base -4096, shift +4096)
        seqs=dict(kind="fixed", seg_lens=[129024], offline=[-4096]),
        n_prefill=2048, n_decode=1,
    ),
    "batch": dict(
        idx=4, n_layers=8, n_kv=8, group=8, head_dim=128, dtype="bf16", page_size=16,
        theta=10000.0, k_scale=1.0,
        mix=[(LOCAL, 85, 256, 0), (GLOBAL, 10, 0, 0), (RETRIEVAL, 5, 0, 32)],
        seqs=dict(kind="random", n_seq=32, len_lo=8192, len_hi=65536,
                  seg_lo=2048, seg_hi=8192, off_lo=0, off_hi=65536),
        n_prefill=256, n_decode=1,
    ),
    # Head-level recovery prefill: the global slots of the 32K workload
    # recomputed in full, every context token a query (causal, one chunk).
    "recovery32k": dict(
        idx=5, n_layers=1, n_kv=10, group=4, head_dim=128, dtype="bf16", page_size=16,
        theta=10000.0, k_scale=0.5,
        slot_classes=[(GLOBAL, 0)] * 10,
        seqs=dict(kind="fixed", seg_lens=[], offline=[]),
        n_prefill=30000, n_decode=1,
    ),
}

ORDER = ["tiny", "32k", "16k", "128k", "batch"]
