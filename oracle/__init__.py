"""CPU oracle for packed variable-length attention (test infrastructure only).

This package is test infrastructure.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The library under
``variable_length_packed_pack_amd/`` never imports it, and the oracle shares no
code with that library: no kernels, no helpers, no constants.

Every function here is a plain, slow, obviously correct restatement of a
definition from the pages:

* ``pack_sequences``      -- "gigl.nn.packed_attention", "Data flow of a packed
                             forward" and "Example".
* ``grid_capacity``       -- "So you wanna CUDA Graph", "Scheduling without
                             max_seqlen" (the launch-capacity bound G_cap).
* ``build_ragged_grid``   -- "PyCoRa", section "CoRa Metadata"; "So you wanna
                             CUDA Graph", "Scheduling without max_seqlen"
                             (chunk_offsets prefix sum and its decode).
* ``decode_tile``         -- the same section's flat-chunk decode.
* ``varlen_attention``    -- "PyCoRa", "Ragged Flash Attention" (exact attention
                             per sequence); "gigl.nn.packed_attention" (each
                             sequence attends only to itself; first-token
                             queries).
* ``cu_seqlens_from_ids`` -- run boundaries of per-token document ids, with a
                             fixed-capacity tail ("So you wanna CUDA Graph",
                             "Terminology time").
* ``document_masked_attention`` -- attention over one packed sequence under
                             the sample-id mask, the dense definition that
                             varlen attention must equal.
* ``ragged_matmul``       -- "PyCoRa", "Ragged Matrix Multiplication" (each
                             sequence times its own weight matrix); a shared
                             weight gives the packed projections of
                             "gigl.nn.packed_attention".
* ``varlen_attention_bwd`` -- the gradient of ``varlen_attention`` (no first-
                             token mode) with respect to q, k and v; the pages
                             train through the packed attention
                             ("gigl.nn.packed_attention", "Why this exists";
                             "DanLing NestedTensor" 3.4) but give no backward
                             algorithm, so this is the derivative written out.

All pins are in ``tests/test_oracle.py``; no oracle function is "parity unpinned".
"""

from .varlen_oracle import (  # noqa: F401
    INT32_MAX,
    build_ragged_grid,
    cu_seqlens_from_ids,
    document_masked_attention,
    decode_tile,
    grid_capacity,
    pack_sequences,
    ragged_matmul,
    varlen_attention,
    varlen_attention_bwd,
    varlen_attention_bwd_rows,
    varlen_attention_rows,
)
