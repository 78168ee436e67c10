"""MI355X-native vision-to-language bridge: k x k space-to-depth merge, two-Linear
GELU projector and placeholder scatter as hand-written HIP kernels for gfx950,
behind the C ABI of include/vlbridge.h (libvlbridge.so) and its Python binding
(patch_merge_mlp_amd.vlbridge)."""
