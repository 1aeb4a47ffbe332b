"""CPU float64 oracle for the LoRA linear layer -- TEST INFRASTRUCTURE ONLY.

Imported by the tests, the smoke check and the benchmark's CPU baseline; the
HIP library and its binding never import it.  See lora_oracle.py for the
definitions and their sources.
"""
from .lora_oracle import *  # noqa: F401,F403
from .lora_oracle import __all__  # noqa: F401
