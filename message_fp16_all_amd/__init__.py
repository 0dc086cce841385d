"""MI355X-native FP16 all-reduce combine.

``hr`` is the Python binding of the C-ABI library ``libhr.so`` (built from
``csrc/``): argument marshalling only, every step runs in the HIP kernels.
``inputs`` draws the seeded synthetic contributions.  Importing this package
loads nothing; ``message_fp16_all_amd.hr`` loads the library on first use.
"""
