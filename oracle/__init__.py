"""fp64 CPU reference for decode attention.  Test infrastructure only: the product
path never imports this package (see oracle.py and decode_oracle.c)."""
