"""CPU oracle for the group-wise low-bit weight-only GEMV (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and the library never imports it.  See :mod:`oracle.wq_oracle` for the
definitions, their sources on the pages, and the readings taken where the
pages are silent.

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (values the pages print, closed forms, library routines,
exhaustive or brute-force checks); none is "parity unpinned".
"""

from .wq_oracle import (  # noqa: F401
    GROUP, CODEBOOK_DECIMAL, CODEBOOK_FP16, CODEBOOK_F64, THRESHOLDS_F64, OLS_EPS,
    quantize_w4, pack_w4, unpack_w4, dequant_w4, pack_zeros_w4, unpack_zeros_w4,
    quantize_w2, pack_w2, unpack_w2, dequant_w2,
    outlier_count, outlier_scores, select_outliers, split_outliers,
    channel_saliency, saliency_kurtosis, kurtosis_ratio, select_outliers_kurtosis,
    KURT_R_BASE, KURT_R_MIN, KURT_R_MAX,
    QuantLayer, quantize_layer, background_mask, matvec_ref,
    REFINE_CHUNK, topk_chunks, refinement_w4, refine_ref,
    TOL_REL, TOL_ABS, check_tolerance, fidelity,
)
