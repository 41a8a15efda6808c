"""Layerwise QK-Norm for AMD Instinct MI355X (gfx950).

The computation lives in libqknorm.so (hand-written HIP kernels behind a C ABI declared in
include/qknorm.h); this package is its thin Python binding plus the seeded input generator.
"""

from ._lib import (QKN_BF16, QKN_F32, QknError, lib, mailbox_epochs, mailbox_values,
                   mailbox_words, normproj_deferred, normproj_deferred_layernorm,
                   normproj_deferred_layernorm_noalloc, normproj_fold_layernorm,
                   normproj_fold_weight, normproj_layernorm_unfused, normproj_unfused,
                   qkn_device_copy, qknorm_apply_with_stats, qknorm_fused, qknorm_partial_sumsq,
                   qknorm_project_eliminated, qknorm_project_unfused, qknorm_shard_fused,
                   qknorm_shard_publish)

__all__ = ["QKN_BF16", "QKN_F32", "QknError", "lib", "mailbox_epochs", "mailbox_values",
           "mailbox_words", "normproj_deferred", "normproj_deferred_layernorm",
           "normproj_deferred_layernorm_noalloc", "normproj_fold_layernorm",
           "normproj_fold_weight", "normproj_layernorm_unfused", "normproj_unfused",
           "qkn_device_copy", "qknorm_apply_with_stats", "qknorm_fused", "qknorm_partial_sumsq",
           "qknorm_project_eliminated", "qknorm_project_unfused", "qknorm_shard_fused",
           "qknorm_shard_publish"]
