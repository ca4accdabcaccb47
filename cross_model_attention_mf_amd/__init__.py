"""MapFlow hot path on MI355X: staged block compression of a sender's attention
map and the fused mapped-attention . V kernel, behind a C ABI (libmapflow.so),
with a prefix cache of compressed maps and the least-squares fit of the head
mapping from compressed maps.

Import `cross_model_attention_mf_amd.mapflow` for the binding; importing the
package itself loads nothing.
"""
