"""MI355X (gfx950) group-wise low-bit weight-only GEMV: W4 (asymmetric uniform,
group 32) and W2 (Lloyd-Max codebook + OLS scale/zero, group 32), each with
FP16 outlier columns, behind the C ABI of ``include/wq.h``.

``_lib`` is the ctypes binding of ``libwq.so`` (same names as the C ABI);
``layer`` packs a float32 weight matrix with the library's host encoder and
moves the packed arrays to the GPU.  Nothing here computes on the CPU except
the library's own host encoder, and nothing falls back to another
implementation: calls fail if ``libwq.so`` has not been built.
"""

from ._lib import (  # noqa: F401
    WQError, load, LIB_PATH, WQ_FMT_W4, WQ_FMT_W2, WQ_FMT_W4P, WQ_FUSE_OUTLIERS, WQ_GROUP, WQ_MAX_K,
    WQ_GEMM_MAX_M, SIGNATURES, VARIANT_FIELDS, Variant, variant,
    wq_quantize_w4, wq_quantize_w2, wq_pack_zeros_w4, wq_select_outliers,
    wq_select_outliers_kurtosis, wq_split_outliers,
    wq_dequant_host, wq_refinement_w4, wq_dequant_device, wq_gemv_w4, wq_gemv_w2, wq_gemv_w4p, wq_gemm_wq,
    wq_outlier_add, wq_embed_gather, wq_topk_count, wq_topk_chunks, wq_refine_add,
    wq_refine_topk,
    wq_tiled_bytes, wq_tile_host, wq_gemv_tiled, wq_gemm_tiled, wq_gemv_tiled_refine,
    wq_read_probe, wq_read_probe_sink_words, wq_read_probe_geom, wq_copy_probe,
)
