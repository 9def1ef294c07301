"""libssd: Mamba-2 SSD chunked scan (forward + backward) for AMD MI355X (gfx950).

The compute path is the HIP library libssd.so (C ABI in include/ssd.h);
`ssd` is its thin Python binding and `inputs` the seeded synthetic inputs.
"""
