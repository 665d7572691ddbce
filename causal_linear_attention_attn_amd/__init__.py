"""Causal linear attention (elu+1 kernel, per-head decay, gated delta rule)
on MI355X: a thin Python binding over the C-ABI library liblinattn.so."""
