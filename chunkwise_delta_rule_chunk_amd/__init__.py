"""MI355X-native chunkwise gated delta rule (DeltaNet / GDN / KDA) with the
ReWY backward.  The operator runs in hand-written gfx950 HIP kernels behind the
C ABI declared in include/rewy.h; this package is the thin Python binding."""
from . import flops  # noqa: F401
