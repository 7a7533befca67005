"""RaZeR-NVFP4 W4A16 for AMD MI355X (gfx950): Python binding of librazer."""
