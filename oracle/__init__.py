"""Oracle: a plain, slow, obviously correct CPU definition of the shard step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import or run anything here; the product
(the C-ABI library and its Python binding) never does, and shares no code
with it.  The oracle is written from the pages' description of DDP gradient
bucketing and ZeRO-1/2/3 sharding (see each function's docstring for the
passage it follows) and from the readings listed with each function where
the pages leave a step open.

Precision.  The pages fix the arithmetic: bf16 gradients and parameters, an
fp32 master weight and fp32 Adam moments, gradients summed in fp32.  So the
oracle computes in IEEE binary32 with one round-to-nearest-even rounding per
operation (numpy float32 ufuncs: one rounding each, no fused multiply-add,
subnormals kept), and host scalars in float64 rounded once to binary32.

Modules:
  plan   bucket plans -- whole tensors per bucket, fixed-size buckets with
         tensors split across them, one bucket per tensor with dim-0 row
         shards -- with per-tensor offsets, padding, per-rank chunks, the
         shard map and model-state byte accounting
  step   pack / unpack / chunk / gather, ascending-rank reduce, accumulate,
         normalise, AdamW, bf16 cast, the whole shard step composed from
         them, global gradient-norm clipping (squared norm, coefficient,
         scale), and parameter groups (per-element groups of a shard, the
         grouped step)

Every function is pinned by tests/test_oracle_*.py against closed forms,
invariants, special cases, library routines or brute force; none is
"parity unpinned".
"""

from . import plan, step  # noqa: F401
