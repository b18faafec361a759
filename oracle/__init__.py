"""Oracle: plain, slow, fp64 CPU definitions of the sequence-parallel attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the ``ltxa`` C ABI, its
HIP kernels, or the Python binding in ``video_dit_sequence_amd``) may import,
call or link anything under this directory.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

The oracle shares no code with the HIP path.  Every function takes numpy arrays
(floating point widened to float64 by the caller, integers as given) and
returns numpy arrays.  Each function names the passage of the source pages it
follows:

* "Sequence Parallelism (SP)" page of LTX-2's multi-GPU docs, sections
  "What it is", "How the forward pass works", "API / AttentionManager" and
  "Usage" -- the pad / shard / head-exchange / global-attention / shuffle-back
  procedure, the byte-exact round trip, head divisibility and ``max_tokens``.
* FastVideo API page ``fastvideo.models.encoders.gemma``, entries
  ``LTXRopeType``, ``apply_ltx_rotary_emb``, ``precompute_ltx_freqs_cis`` and
  the ``Embeddings1DConnector`` forward -- interleaved rotary embedding over
  (t, x, y) positions normalised by ``max_pos`` with base ``theta``.

Where the pages are silent the oracle takes one stated reading; each reading
is listed in the module that uses it.

Parity status:
* ``perm``  -- pinned (hand-written fixture, numpy transpose, round trip).
* ``rope``  -- pinned by closed forms and invariants.  The frequency schedule
  itself is a reading (the page prints the function signatures only), so its
  agreement with upstream LTX-2 numerics is *parity unpinned*; the schedule
  used here is pinned to its own closed form.  The variants (split pairing,
  grid over the inner dimension, middle indices) are readings too, pinned to
  hand-derived angles and to identities that reduce each to the base case.
* ``attn``  -- pinned by brute force, closed forms and invariants.
"""

from .perm import sp_pack, sp_unpack, pad_length
from .rope import rope_angles, rope_apply
from .attn import attention
from .path import sp_path_single_gpu, sp_path_virtual_ranks

__all__ = [
    "sp_pack", "sp_unpack", "pad_length",
    "rope_angles", "rope_apply",
    "attention",
    "sp_path_single_gpu", "sp_path_virtual_ranks",
]
