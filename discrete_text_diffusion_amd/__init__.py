"""MI355X (gfx950) canvas denoise step of DiffusionGemma-style discrete text diffusion.

    from discrete_text_diffusion_amd import dg        # ctypes binding of include/dg.h
    from discrete_text_diffusion_amd.model import Model

The HIP library (libdg.so) is built in-tree by discrete_text_diffusion_amd.build.build().
"""
__all__ = ["dg", "model", "build"]
