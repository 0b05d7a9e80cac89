"""Location of the built library (kept apart so importing it builds nothing)."""
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmoe_layout.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
