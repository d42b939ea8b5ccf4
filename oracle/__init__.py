"""Plain fp64 CPU oracle for the routed-expert MXFP4 MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP library (``mxfp4_mixture_experts_moe_amd``), and the
library never imports it.

It is written straight from the definitions on the pages it cites, in the
simplest form a reader can check by eye: numpy in fp64, with library
primitives (matmul, stable sort) as single steps and no blocking or fusion.

Modules
-------
``mxfp4``   the two MXFP4 block encodings: source decode, repack, ggml dequant
``route``   sigmoid + bias top-k routing
``permute`` stable grouping of (token, slot) entries by expert
``ffn``     the routed-expert FFN: route -> per-expert SiLU-gated MLP -> weighted sum
``verify``  expert bytes of a speculative verify batch by width, and the width a cost hint picks
``cache``   a least-recently-used device expert cache in front of an external expert store
``latent``  the latent-MoE block: gate projection, latent down + RMS norm, routed
            experts, latent up, shared expert
``q4k``     Q4_K expert blocks (ggml's 4-bit k-quant): decode, and the routed FFN
            over Q4_K experts

Parity status
-------------
Every function here is pinned by ``tests/test_oracle_*.py`` against something
other than itself (values printed on the pages, IEEE-754 closed forms, a
library decode of E8M0, a textbook sort, brute-force loops, an identity-weight
closed form, a hand-worked verify-width choice, a hand-worked cache sequence
and an independent last-use LRU simulation, bf16 rounding against every bf16
value and torch's conversion, an identity-weight closed form of the latent
block and its pure-Python loop evaluation).  The FFN's numerics beyond those closed forms have no worked
example on the pages; ``ffn_ref`` is pinned by a pure-Python loop evaluation
and the identity case only.  The pages name Q4_K without defining it:
``q4k`` follows ggml's published block layout and is pinned to a hand-encoded
block, an inverse-packing round trip over every 6-bit value, fp16 closed
forms and a pure-Python loop evaluation of the FFN on design values, none of
which the pages can confirm.
"""

from .mxfp4 import (  # noqa: F401
    E2M1,
    KVALUES,
    decode_ct,
    dequant_ref,
    repack_ref,
    source_codes,
    unrepack_ref,
)
from .route import route_ref  # noqa: F401
from .permute import permute_ref, valid_entries  # noqa: F401
from .ffn import ffn_ref, silu_mul  # noqa: F401
from .verify import expected_committed, verify_distinct_ref, verify_width_choose_ref  # noqa: F401
from .cache import ExpertCacheRef  # noqa: F401
from .latent import bf16_round, latent_block_ref, rms_norm  # noqa: F401
from .q4k import ffn_q4k_ref, q4k_codes, q4k_decode, q4k_scale_min  # noqa: F401
