"""MI355X-native dynamically quantized int8 linear layer (W8A8, dense + BSR).

The HIP library (libw8a8.so, C ABI in include/w8a8.h) does all the work; the
Python module `binding` only marshals torch tensors into it. Importing this
package loads nothing: call `binding.load()` (done lazily by every entry point),
which raises if the library has not been built.
"""
