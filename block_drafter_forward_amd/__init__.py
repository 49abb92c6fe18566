"""MI355X (gfx950) block drafter forward: HIP kernels behind a C ABI (include/fm.h) and a thin ctypes binding.

    from block_drafter_forward_amd import fm
    d = fm.Drafter(cfg, fm.upload_weights(weights))
    d.fm_context_append(taps, start=0)
    d.fm_draft_block(hidden, anchor=anchor_dev, pos=n)
    d.fm_lm_argmax(hidden, rows, tokens)
"""
