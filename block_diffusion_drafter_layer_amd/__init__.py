"""DFlash drafter hot path on MI355X (gfx950): HIP kernels behind a C ABI.

    from block_diffusion_drafter_layer_amd import binding   # loads libdflash.so
    from block_diffusion_drafter_layer_amd.drafter import Drafter

Build the library first with ``python -m block_diffusion_drafter_layer_amd.build``;
importing ``binding`` raises ImportError when it is missing.
"""
