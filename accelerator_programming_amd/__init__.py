"""MI355X-native (gfx950) tiled fused attention forward.

The compute path is a hand-written HIP library (``csrc/``) behind a C ABI
(``include/attn_fwd.h``); ``attn`` is its thin ctypes binding. Importing this
package loads nothing; the binding loads the library on first use and raises
if it has not been built.
"""
