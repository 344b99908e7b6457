"""CPU oracle for the HeadQ key-side KV cache — test infrastructure only (see oracle.py)."""
