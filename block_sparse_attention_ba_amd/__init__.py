"""MI355X-native Block Approximate Sparse Attention (BA-Att).

`api` holds the Python binding of the HIP library (select, forward, dense,
mask_to_index); `workloads` the seeded synthetic inputs.  Importing the
package loads nothing: the HIP library is loaded on first use and its absence
is an error.
"""

__version__ = "0.1.0"
