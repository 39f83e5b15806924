"""Placeholder until the HIP library exists."""
__all__ = []
