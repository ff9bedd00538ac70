"""CPU oracle for the strict joint-attention path (test infrastructure only)."""
from .oracle import Oracle, build, fold_batch, forward_path, qkv_path  # noqa: F401
