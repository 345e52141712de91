"""MI355X-native Barnes-Hut force evaluation (HIP, gfx950).

The evaluation runs in liborr.so (C ABI in include/orr.h); ``orr`` is its
Python binding and ``inputs`` the seeded workload generators. Importing the
package loads neither torch nor the library; ``orr`` does both when imported.
"""

__all__ = ["inputs", "orr"]
