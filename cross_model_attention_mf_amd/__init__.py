"""MapFlow hot path on MI355X: staged block compression of a sender's attention
map and the fused mapped-attention . V kernel, behind a C ABI (libmapflow.so).

Import `cross_model_attention_mf_amd.mapflow` for the binding; importing the
package itself loads nothing.
"""
