"""ctypes binding of the C-ABI library (filled in with the library)."""
__all__ = []
