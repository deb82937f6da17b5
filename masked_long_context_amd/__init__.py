"""MI355X-native BDLM-masked core attention (bdattn): forward, backward, LSE
merge and varlen packed-shard attention in hand-written gfx950 HIP kernels
behind a C ABI.  The HIP binding is loaded lazily by ``masked_long_context_amd.bdattn``."""
