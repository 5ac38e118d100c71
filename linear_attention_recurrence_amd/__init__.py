"""MI355X (gfx950) implementation of the KDA gated delta-rule recurrence.

The compute lives in libkda.so (hand-written HIP kernels behind the C ABI of
include/kda.h); this package is its thin Python binding. torch provides
device memory and streams only.
"""
from .kda import (  # noqa: F401
    KDA_BF16, KDA_CHUNK, KDA_ERR_DEVICE, KDA_ERR_HOST_ALLOC, KDA_ERR_INVALID_ARG, KDA_ERR_NO_SLOT, KDA_ERR_UNSUPPORTED,
    KDA_SLOT_FREE, KDA_SLOT_TREE, RequestSlots, SlotPool, kda_chunk_split, kda_decode, kda_state_move,
    KDA_F32, KDA_HEAD_DIM, KDA_OK, KDA_PLAN_FIFO, KDA_PLAN_LPT, KDA_PREFILL_PLAN_RESIDENT, EXPORTS, KdaError,
    Plan, Ring, kda_abi_version, kda_chunk_prefill, kda_chunk_prefill_gated, kda_gated_rmsnorm, kda_last_error, kda_prologue, kda_plan_create, kda_plan_items,
    kda_fold_verify, kda_plan_num_items, kda_plan_upload, kda_plan_v_blocks, kda_plan_workspace_bytes,
    KDA_NOALLOC_SCRATCH_BYTES, kda_chunk_prefill_noalloc, kda_host_release, kda_replay_fold, kda_verify, kda_verify_ragged, lib,
    kda_probe_copy, kda_probe_mfma, kda_probe_read,
)
