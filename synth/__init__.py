"""Seeded synthetic inputs for the calibrated block-sparse attention path.

This package only draws random numbers and lays out input structure
(tensor shapes, video token grids, block masks of a given density). It holds
none of the method's arithmetic: no softmax, no energy, no selection, no
mask compilation. Both the fp64 oracle and the HIP path receive the arrays it
returns.
"""

from .inputs import *  # noqa: F401,F403
