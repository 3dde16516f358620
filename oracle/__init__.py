"""CPU oracle for the GLM-5.3-Flash DSA decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package; only the tests, the package smoke check and the bench's CPU
baseline leg do.  It shares no code with the HIP library.

Every function is a plain fp64 numpy restatement of one step as the Atlas
``glm5next_dsa`` page states it (its "Shape of the pipeline" diagram and its
"Traps carried from Slice 8" list), plus the fp32 head-gate product of the
stkernel PR #227 page.  Readings of points the pages leave open are stated in
each docstring.
"""
from .dsa_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    fp8_e4m3_to_f64,
    head_gate,
    kpool_geometry,
    kpool_compress,
    request_rows,
    layer_norm_rows,
    indexer_store,
    write_geom,
    slot_weights,
    index_scores,
    topk_pools,
    expand_selection,
    select_tail,
    sparse_mla_decode,
    sparse_mla_decode_paged,
    latent_rows_f64,
    paged_rows,
    kv_index,
    attend_rows,
    select_k,
    out_width,
    dsa_step,
)
