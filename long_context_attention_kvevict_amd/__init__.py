"""MI355X-native windowed KV-cache eviction: score, select, compact and
SNIS decode, as a C-ABI HIP library (libkvevict.so) with a thin ctypes
binding.  PyTorch is used only for device memory and streams."""

__all__ = ["synth", "workloads"]
