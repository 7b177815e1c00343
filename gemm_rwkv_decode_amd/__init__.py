"""Placeholder; replaced by the binding below once the C-ABI exists."""
