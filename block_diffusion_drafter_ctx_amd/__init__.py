"""MI355X-native DFlash drafter hot path: HIP kernels behind a C-ABI library.

``block_diffusion_drafter_ctx_amd.binding`` loads ``libdflash.so`` (built by
``__graft_entry__.build()``) and exposes its four calls; ``roofline`` holds the
algorithmic byte / flop accounting used by the benchmark.
"""
__all__ = ["binding", "roofline"]
