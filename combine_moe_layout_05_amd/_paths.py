"""Location of the built library (kept apart so importing it builds nothing)."""
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmoe_layout.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# Traffic reference kernels the benchmark runs beside the combine (not part
# of the library's C ABI).
PROBE_LIB_NAME = "libmoe_traffic_probe.so"
PROBE_LIB_PATH = os.path.join(PKG, PROBE_LIB_NAME)
