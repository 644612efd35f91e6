"""Seeded synthetic inputs for the low-bit weight-only GEMV workloads.

This module only draws random numbers and shapes them: float32 weight
matrices, FP16 activation vectors, spike-channel sets and activation
profiles.  It holds none of the method's arithmetic (no quantization, no
packing, no outlier selection, no products).  Both the CPU oracle side
(tests, the CPU baseline) and the GPU side (tests, bench) draw their inputs
from here, so that the two see identical host arrays.

Seeds: every array comes from
``np.random.default_rng(np.random.SeedSequence([2026, cfg, layer, proj, role]))``
with role 0 = W, 1 = x, 2 = per-group mean shift, 3 = spike set, 4 = profile.

The workloads stand in for the trained layers the pages quantize (there are
no checkpoints here): i.i.d. Gaussian weights at the shapes of the models the
pages name, FP16 Gaussian activations, and a few channels scaled up to mimic
the activation spikes described on the OTF-LLM v4.0 page, section 4
("Profile-Guided Activation Outliers").
"""

from .workloads import (  # noqa: F401
    ROLE_W, ROLE_X, ROLE_SHIFT, ROLE_SPIKES, ROLE_PROFILE,
    rng_for, gaussian_weights, gaussian_x_fp16, spike_set,
    Layer, small_layer, config1, config2, config3_shapes, config3_layer,
    config4, config5, LLAMA3_8B_SWEEP, OUTLIER_RATIO,
)
