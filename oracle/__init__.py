"""fp64 CPU oracle for ring-order block attention and the Ulysses transposes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It imports nothing from ``ring_ulysses_sequence_amd``
and shares no code with the HIP kernels.  Everything here is plain, slow and
written to be checked against the pages by eye.

Sources (the pages this follows, cited by title and section):

* "序列并行与 Ring Attention" (Sequence Parallelism and Ring Attention
  tutorial, jefxiong.cn) -- §3.1 scaled dot-product attention and the rank-local
  output, §3.2 the online-softmax recurrence over (m, l, u), §3.3 the ring order
  (source (r - t) mod P at round t), §3.4 causal block classes on global
  positions and the zigzag load-balancing idea, §3.5 the Ulysses seq-shard <->
  head-shard transpose, §6.2 the ring backward, §6.6 the fp64 gradient oracle, §04 the
  4 x 2 worked example, §09 the stability and global-index checks.
* juejin post 7702110021828427786 (a sequence-parallel attention library that
  never communicated) -- §三 the shard-cover and did-it-communicate checks,
  §四 the log-sum-exp combine and the is_causal precondition on skipping,
  §五 the chunked-merge unit test.
* "Finalize guidelines for Ulysses-based context-parallel attention"
  (aitangshan.cn) -- §三/§四/§六/§七 padding the sequence to a multiple of P.
* "多卡通算融合算子精度校验" (fused comm+compute precision checks,
  triton-distributed-ascend) -- §3.1 golden in higher precision, §3.4 dtype
  tolerance tiers, integers bit-exact.

Parity status of each function is listed in its module docstring.
"""
from .attention import attention, local_only_attention, scores, gqa_expand, packed_attention
from .online import (ring_attention_rank, lse_combine, composable_ring_rank, chunked_attention,
                     zigzag_ring_rank)
from .schedule import (SKIP, FULL, DIAG, padded_len, seq_divisible, shard_range, ring_sources,
                       classify_block, ring_schedule, visible_mask, zigzag_chunks,
                       zigzag_positions, zigzag_schedule, visible_pairs)
from .permute import seq2head, head2seq, seq2head_loops, head2seq_loops
from .grad import attention_grad, attention_grad_sampled, ring_attention_bwd_rank
from .compare import max_abs_err, cosine, rel_l2, compare

__all__ = [
    "attention", "local_only_attention", "scores", "gqa_expand", "packed_attention",
    "ring_attention_rank", "lse_combine", "composable_ring_rank", "chunked_attention",
    "zigzag_ring_rank", "zigzag_chunks", "zigzag_positions", "zigzag_schedule", "visible_pairs",
    "attention_grad", "attention_grad_sampled", "ring_attention_bwd_rank",
    "SKIP", "FULL", "DIAG", "padded_len", "seq_divisible", "shard_range", "ring_sources",
    "classify_block", "ring_schedule", "visible_mask",
    "seq2head", "head2seq", "seq2head_loops", "head2seq_loops",
    "max_abs_err", "cosine", "rel_l2", "compare",
]
